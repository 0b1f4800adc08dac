"""GPU parity of the gate W_g (gamma = sigmoid(g) on the linear branch inside
the shared normaliser; list view Table 9, full text Sec. 4.1 and App. A.6.1)
against the float64 oracle: the forward on both kernel paths, the prefill ->
decode hand-off and decode steps on both decode paths, and the backward
including the gate logits' gradient.  Bars as for the ungated operator:
selections exact (or near-ties the oracle adopts), outputs rel-L2 <= 1e-2
(bf16) / 1e-5 (fp32) and every row within its per-row bar, gradients
rel-L2 <= 1e-4."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import (BF16_TOL, F32_TOL, check_rows, check_selection, make_case, prepare, rel_l2,
                    row_tol, say, torch_dtype)

pytestmark = pytest.mark.gpu

FWD_CASES = {
    "bf16_G4": (make_case("a", 2, 333, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 81),
    "bf16_G2": (make_case("b", 1, 300, 4, 2, 128, 64, 64, 8), 82),
    "f32_d64_W48_C16": (make_case("c", 1, 150, 4, 1, 64, 48, 16, 4, dtype="f32"), 83),
    "bf16_swa_la": (make_case("d", 1, 200, 4, 2, 128, 64, 64, 0), 84),
    "bf16_W128_G4": (make_case("j", 1, 400, 8, 2, 128, 128, 64, 16), 90),
    "bf16_W128_C128_G4": (make_case("k", 1, 450, 8, 2, 128, 128, 128, 16), 91),
}


def gate_tensor(cfg, seed, kind):
    g = workloads.make_gate(cfg, seed)
    if kind == "closed":
        g[:] = -np.inf
    elif kind == "open":
        g[:] = np.inf
    return g


@pytest.mark.parametrize("kind", ["random", "closed"])
@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(FWD_CASES))
def test_gated_fwd_matches_oracle(gpu_lib, name, general, kind):
    cfg, seed = FWD_CASES[name]
    say(f"[gate fwd] case={name} general={general} gate={kind} shape={workloads.shape_of(cfg)}")
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    gl = gate_tensor(cfg, seed, kind)
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                      topk=lam, return_sel=True, general=general, gate=torch.from_numpy(gl).cuda())
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam)
    sigma = O.window_scores(ref["q"], ref["k"], p, cfg["n_kv_heads"]) if W > 0 else None
    override = None
    if p.topk_eff() > 0:
        osel, _ = O.select_chunks(sigma, p)
        gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
        if check_selection(gsel, sigma, osel, C)[0]:
            override = gsel
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p,
                     sel_override=override, scores=sigma, gate=gl)
    out = res["out"].double().cpu().numpy()
    assert np.isfinite(out).all()
    err = rel_l2(out, o["out"])
    tol = F32_TOL if cfg["dtype"] == "f32" else BF16_TOL
    say(f"  out rel-L2 {err:.3e} (tol {tol:g})")
    assert err <= tol
    check_rows(out, o["out"], row_tol(cfg["dtype"]))


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
def test_open_gate_equals_ungated_bit_for_bit(gpu_lib, general):
    """gamma = sigmoid(+inf) = 1 exactly, so the gated kernels must return
    exactly what they return without a gate."""
    cfg, seed = FWD_CASES["bf16_G4"]
    raw = workloads.make_prefill(cfg, seed)
    dev, _ = prepare(raw, torch.bfloat16)
    kw = dict(window=64, chunk=64, topk=16, general=general)
    a = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], **kw)["out"]
    g = torch.from_numpy(gate_tensor(cfg, seed, "open")).cuda()
    b = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], gate=g, **kw)["out"]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


DEC_CASES = {
    "bf16_G4": (make_case("e", 2, 130 + 70, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 130, 85),
    "f32_W48_C16": (make_case("f", 1, 70 + 40, 4, 1, 64, 48, 16, 4, dtype="f32"), 70, 86),
}


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(DEC_CASES))
def test_gated_prefill_then_decode(gpu_lib, name, general):
    cfg, N0, seed = DEC_CASES[name]
    say(f"[gate decode] case={name} general={general} shape={workloads.shape_of(cfg)} N0={N0}")
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    gl = workloads.make_gate(cfg, seed)
    gd = torch.from_numpy(gl).cuda()
    B, N, Hkv, d = cfg["batch"], cfg["seqlen"], cfg["n_kv_heads"], cfg["head_dim"]
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    p = O.Params(window=W, chunk=C, topk=lam)
    cap = p.topk_eff() * (-(-N // C)) + 1
    tol = F32_TOL if cfg["dtype"] == "f32" else BF16_TOL
    gc = gpu_lib.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C, topk=lam,
                             sel_cap=cap, dtype=dt, pos=N0)
    res = gpu_lib.fwd(dev["q"][:, :N0].contiguous(), dev["k"][:, :N0].contiguous(),
                      dev["v"][:, :N0].contiguous(), dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                      topk=lam, return_sel=True, cache=gc, general=general,
                      gate=gd[:, :N0].contiguous())
    torch.cuda.synchronize()
    sig = O.window_scores(ref["q"][:, :N0], ref["k"][:, :N0], p, Hkv)
    osel, _ = O.select_chunks(sig, p)
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    override = gsel if check_selection(gsel, sig, osel, C)[0] else None
    o_pre, oc = O.fwd_recurrent(ref["q"][:, :N0], ref["k"][:, :N0], ref["v"][:, :N0], ref["wphi_q"],
                                ref["wphi_k"], p, cap=cap, sel_override=override, gate=gl[:, :N0])
    out = res["out"].double().cpu().numpy()
    assert rel_l2(out, o_pre) <= tol
    check_rows(out, o_pre, row_tol(cfg["dtype"]), what="prefill")
    worst = 0.0
    for t in range(N0, N):
        g_out = gpu_lib.decode_step(dev["q"][:, t:t + 1].contiguous(), dev["k"][:, t:t + 1].contiguous(),
                                    dev["v"][:, t:t + 1].contiguous(), dev["wphi_q"], dev["wphi_k"], gc,
                                    general=general, gate=gd[:, t:t + 1].contiguous())
        o_out = O.decode_step(oc, ref["q"][:, t], ref["k"][:, t], ref["v"][:, t], ref["wphi_q"],
                              ref["wphi_k"], p, gate_t=gl[:, t])
        torch.cuda.synchronize()
        g_np = g_out[:, 0].double().cpu().numpy()
        err = rel_l2(g_np, o_out)
        worst = max(worst, err)
        assert err <= tol, f"step t={t}: rel-L2 {err:.3e}"
        check_rows(g_np, o_out, row_tol(cfg["dtype"]), what=f"step t={t}")
        if t % C == C - 1 and lam > 0:
            # chunk-end decisions: the same flags, or a near-tie the oracle adopts
            gf = gc.win_route.cpu().numpy()
            slots = [j % W for j in range(t - C + 1, t + 1)]
            if not np.array_equal(gf[:, :, slots], oc["win_route"][:, :, slots]):
                pos = np.arange(t - C + 1, t + 1)
                for b in range(B):
                    for g in range(Hkv):
                        gs = pos[gf[b, g, slots] == O.ROUTE_SA][None, None, None, :]
                        os_ = pos[oc["win_route"][b, g, slots] == O.ROUTE_SA][None, None, None, :]
                        sg = np.zeros((1, 1, t + 1))
                        sg[0, 0, pos] = oc["pend_score"][b, g, pos % C]
                        check_selection(gs, sg, os_, C)
                oc["win_route"][:, :, slots] = gf[:, :, slots]
    say(f"  {N - N0} gated steps, worst rel-L2 {worst:.3e}")


BWD_CASES = {
    "bf16_G4": (make_case("g", 1, 300, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 87),
    "f32_d64_W48_C16": (make_case("h", 1, 150, 4, 1, 64, 48, 16, 4, dtype="f32"), 88),
    "bf16_swa_la": (make_case("i", 1, 200, 4, 2, 128, 64, 64, 0), 89),
    "bf16_W128_C128_G4": (make_case("l", 1, 450, 8, 2, 128, 128, 128, 16), 92),
}


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(BWD_CASES))
@pytest.mark.parametrize("saved", [0, 1, 2], ids=["recompute", "from_fwd_stats", "from_fwd_stats_ws"])
def test_gated_bwd_matches_oracle(gpu_lib, name, general, saved):
    """saved: the backward starts from the gated forward's output and
    statistics (the gate weight enters the features the dq kernel forms and
    the linear weight c the forward wrote); 2: and from the forward's
    workspace (its keys' features and linear prefixes)."""
    from test_gpu_backward import grad_tol
    cfg, seed = BWD_CASES[name]
    say(f"[gate bwd] case={name} general={general} saved={saved} shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    gl = workloads.make_gate(cfg, seed)
    gd = torch.from_numpy(gl).cuda()
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(dt)
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    sel = None
    fw = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                     topk=lam, return_sel=min(lam, C) > 0, return_stats=saved > 0, gate=gd,
                     return_workspace=saved == 2)
    if min(lam, C) > 0:
        sel = fw["sel_idx"]
    extra = dict(out=fw["out"], stats=fw["stats"]) if saved else {}
    if saved == 2:
        extra["fwd_workspace"] = fw["workspace"]
    g = gpu_lib.bwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], sel, dout.cuda(),
                    window=W, chunk=C, topk=lam, gate=gd, general=general, **extra)
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam)
    o = O.bwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], dout.double().numpy(),
                     p, sel_idx=None if sel is None else sel.cpu().numpy().astype(np.int64), gate=gl)
    errs = {}
    for gname, oname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dwphi_q", "dwq"),
                         ("dwphi_k", "dwk"), ("dgate", "dgate")):
        x = g[gname].double().cpu().numpy()
        assert np.isfinite(x).all(), gname
        errs[gname] = rel_l2(x, o[oname])
    say("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= grad_tol(cfg, general), (k, v)
