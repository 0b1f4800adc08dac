"""GPU parity of the prefill -> decode hand-off and of the decode step against
the oracle's recurrent form (Sec. 3.3 "Recurrent Form"): the cache the
forward leaves behind must equal the oracle's cache after the same tokens,
and each decode step must match the oracle's step, including the chunk-end
routing decisions."""
import copy

import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import (BF16_TOL, F32_TOL, TIE_TOL, check_rows, check_selection, make_case, prepare,
                    rel_l2, row_tol, say, torch_dtype)

pytestmark = pytest.mark.gpu

DEC_CASES = {
    # name: (cfg over N0 + K tokens, N0 prefill tokens, seed)
    "bf16_G4": (make_case("a", 2, 190 + 80, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 190, 31),
    "f32_W48_C16": (make_case("b", 1, 70 + 40, 4, 1, 64, 48, 16, 4, dtype="f32"), 70, 32),
    "bf16_pure_linear": (make_case("c", 1, 20 + 30, 4, 2, 64, 0, 8, 0), 20, 33),
    "bf16_swa_la": (make_case("d", 1, 100 + 40, 4, 4, 128, 32, 64, 0), 100, 34),
    "bf16_from_empty": (make_case("e", 1, 140, 4, 1, 128, 64, 64, 16), 0, 35),
    "bf16_G8_boundary": (make_case("f", 1, 128 + 70, 8, 1, 128, 64, 64, 8), 128, 36),
    # window wider than the chunk, two query heads per KV head (bf16 d=128 decode path)
    "bf16_W48_C16_G2": (make_case("g", 2, 90 + 60, 4, 2, 128, 48, 16, 4, outlier_frac=0.03, heavy_scale=6.0), 90, 37),
    "bf16_W64_C32_G1": (make_case("h", 1, 100 + 50, 2, 2, 128, 64, 32, 8), 100, 38),
    # keys x80 at 3% of positions: logits far beyond 2^128 in exp2 units in
    # both the prefill and the decode steps
    "bf16_huge_logits_G4": (make_case("i", 1, 200 + 60, 8, 2, 128, 64, 64, 16, outlier_frac=0.03,
                                      heavy_scale=80.0), 200, 39),
    # every logit far below -100 (queries along +56 u, keys along -56 u): the
    # steps without a linear term (every routed token selected; the first
    # chunks) must keep their softmax finite
    "bf16_underflow_all_selected": (make_case("u", 1, 150 + 70, 8, 2, 128, 64, 64, 64, anti_align=56.0),
                                    150, 40),
    "bf16_underflow_G4": (make_case("v", 1, 40 + 100, 8, 2, 128, 64, 64, 16, anti_align=56.0), 40, 41),
    # two-chunk window (W = 128, C = 64): matrix-core prefill, then the steps
    "bf16_W128_C64_G4": (make_case("x", 1, 330 + 70, 8, 2, 128, 128, 64, 16), 330, 43),
    "bf16_W256_C64_G2": (make_case("y", 1, 450 + 70, 4, 2, 128, 256, 64, 8), 450, 44),
    # chunks of 128 / 256 tokens: the matrix-core prefill (per-chunk selection,
    # 64-token tiles after it) hands off mid-chunk; decode crosses chunk ends
    "bf16_W128_C128_G4": (make_case("z", 1, 390 + 140, 8, 2, 128, 128, 128, 16), 390, 47),
    "bf16_W256_C256_G2": (make_case("z", 1, 600 + 180, 4, 2, 128, 256, 256, 40), 600, 48),
    "f32_underflow_d64": (make_case("w", 1, 60 + 40, 4, 1, 64, 32, 16, 16, dtype="f32", anti_align=48.0),
                          60, 42),
}


def compare_cache(gc, oc, cfg, n_tok, tol):
    """gc: DecodeCache on the GPU; oc: oracle cache dict.  Exact for copies,
    route flags and counts; tolerance for fp32 sums."""
    W, C = cfg["window"], cfg["chunk"]
    if W > 0:
        n_ring = min(n_tok, W)
        slots = [j % W for j in range(n_tok - n_ring, n_tok)]
        gk = gc.win_k.double().cpu().numpy()
        gv = gc.win_v.double().cpu().numpy()
        np.testing.assert_array_equal(gk[:, :, slots], oc["win_k"][:, :, slots])
        np.testing.assert_array_equal(gv[:, :, slots], oc["win_v"][:, :, slots])
        np.testing.assert_array_equal(gc.win_route.cpu().numpy()[:, :, slots],
                                      oc["win_route"][:, :, slots])
        open_ = [j % C for j in range((n_tok // C) * C, n_tok)]
        if open_:
            gp = gc.pend_score.cpu().numpy()[:, :, open_]
            op = oc["pend_score"][:, :, open_]
            assert np.max(np.abs(gp - op) / np.maximum(1, np.abs(op))) <= 1e-4
    if cfg["topk"] > 0:
        cnt = gc.sel_count.cpu().numpy()
        np.testing.assert_array_equal(cnt, oc["sel_count"])
        gsk = gc.sel_k.double().cpu().numpy()
        gsv = gc.sel_v.double().cpu().numpy()
        for b in range(cnt.shape[0]):
            for g in range(cnt.shape[1]):
                n = cnt[b, g]
                np.testing.assert_array_equal(gsk[b, g, :n], oc["sel_k"][b, g, :n])
                np.testing.assert_array_equal(gsv[b, g, :n], oc["sel_v"][b, g, :n])
    es = rel_l2(gc.lin_S.double().cpu().numpy(), oc["lin_S"]) if np.any(oc["lin_S"]) else \
        float(np.abs(gc.lin_S.cpu().numpy()).max())
    ez = rel_l2(gc.lin_z.double().cpu().numpy(), oc["lin_z"]) if np.any(oc["lin_z"]) else \
        float(np.abs(gc.lin_z.cpu().numpy()).max())
    assert es <= tol and ez <= tol, (es, ez)


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(DEC_CASES))
def test_prefill_handoff_then_decode(gpu_lib, name, general):
    cfg, N0, seed = DEC_CASES[name]
    say(f"[decode] case={name} general={general} shape={workloads.shape_of(cfg)} N0={N0} seed={seed}")
    run_handoff_decode(gpu_lib, cfg, N0, seed, general)


# Budget certification past N_max (full text App. A.4): the quota re-derived
# from the deployment length, lambda(N) = floor((m - W) / ceil(N / C)), keeps
# the selected cache within m - W rows for N > N_max.  The cache is given
# exactly m - W rows; the prefill and every decode step to N must fit.
BUDGET_CASES = {
    # name: (m, N_max, cfg without topk, N0, seed)
    "bf16_d128": (64 + 80, 320, make_case("j", 1, 640, 4, 2, 128, 64, 64, 0), 560, 45),
    "f32_d64": (16 + 64, 128, make_case("k", 1, 256, 2, 1, 64, 16, 16, 0, dtype="f32"), 200, 46),
}


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(BUDGET_CASES))
def test_budget_past_n_max(gpu_lib, name, general):
    m, n_max, base, N0, seed = BUDGET_CASES[name]
    W, C, N = base["window"], base["chunk"], base["seqlen"]
    lam_static = gpu_lib.topk_for_budget(m, W, C, n_max)
    lam = gpu_lib.topk_for_budget(m, W, C, N)
    assert lam == O.topk_for_budget(m, W, C, N) and 0 < lam < lam_static
    cfg = dict(base, topk=lam)
    say(f"[budget] case={name} general={general} m={m} N_max={n_max} N={N} topk {lam_static} -> {lam}")
    run_handoff_decode(gpu_lib, cfg, N0, seed, general, cap=m - W)


def run_handoff_decode(gpu_lib, cfg, N0, seed, general, cap=None):
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    B, N = cfg["batch"], cfg["seqlen"]
    Hq, Hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    p = O.Params(window=W, chunk=C, topk=lam)
    if cap is None:
        cap = p.topk_eff() * (-(-N // C)) + 1
    tol = F32_TOL if cfg["dtype"] == "f32" else BF16_TOL
    state_tol = 1e-5

    gc = gpu_lib.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C, topk=lam,
                             sel_cap=cap, dtype=dt, pos=N0)
    override = None
    if N0 > 0:
        res = gpu_lib.fwd(dev["q"][:, :N0].contiguous(), dev["k"][:, :N0].contiguous(),
                          dev["v"][:, :N0].contiguous(), dev["wphi_q"], dev["wphi_k"], window=W,
                          chunk=C, topk=lam, return_sel=True, cache=gc, general=general)
        torch.cuda.synchronize()
        if p.topk_eff() > 0 and N0 >= C:
            sig = O.window_scores(ref["q"][:, :N0], ref["k"][:, :N0], p, Hkv)
            osel, _ = O.select_chunks(sig, p)
            gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
            if check_selection(gsel, sig, osel, C)[0]:
                override = gsel
    _, oc = O.fwd_recurrent(ref["q"][:, :N0], ref["k"][:, :N0], ref["v"][:, :N0], ref["wphi_q"],
                            ref["wphi_k"], p, cap=cap, sel_override=override)
    compare_cache(gc, oc, cfg, N0, state_tol)
    say("  hand-off cache matches")

    ws = None
    worst = 0.0
    for t in range(N0, N):
        q_t = dev["q"][:, t:t + 1].contiguous()
        k_t = dev["k"][:, t:t + 1].contiguous()
        v_t = dev["v"][:, t:t + 1].contiguous()
        g_out = gpu_lib.decode_step(q_t, k_t, v_t, dev["wphi_q"], dev["wphi_k"], gc,
                                    general=general)
        o_out = O.decode_step(oc, ref["q"][:, t], ref["k"][:, t], ref["v"][:, t], ref["wphi_q"],
                              ref["wphi_k"], p)
        torch.cuda.synchronize()
        assert gc.pos == oc["pos"] == t + 1
        g_np = g_out[:, 0].double().cpu().numpy()
        assert np.isfinite(g_np).all(), f"step t={t}: non-finite output"
        err = rel_l2(g_np, o_out)
        worst = max(worst, err)
        assert err <= tol, f"step t={t}: rel-L2 {err:.3e}"
        check_rows(g_np, o_out, row_tol(cfg["dtype"]), what=f"step t={t}")
        if W > 0 and t % C == C - 1 and lam > 0:
            # chunk-end decision: same flags, or a near-tie that the oracle adopts
            gf = gc.win_route.cpu().numpy()
            slots = [j % W for j in range(t - C + 1, t + 1)]
            if not np.array_equal(gf[:, :, slots], oc["win_route"][:, :, slots]):
                pend = oc["pend_score"]
                for b in range(B):
                    for g in range(Hkv):
                        pos = np.arange(t - C + 1, t + 1)
                        gs = pos[gf[b, g, slots] == O.ROUTE_SA][None, None, None, :]
                        os_ = pos[oc["win_route"][b, g, slots] == O.ROUTE_SA][None, None, None, :]
                        sig = np.zeros((1, 1, t + 1))
                        sig[0, 0, pos] = pend[b, g, pos % C]
                        check_selection(gs, sig, os_, C, TIE_TOL)
                oc["win_route"][:, :, slots] = gf[:, :, slots]
    say(f"  {N - N0} steps, worst step rel-L2 {worst:.3e}")
    compare_cache(gc, oc, cfg, N, state_tol)
    if lam > 0:
        assert int(gc.sel_count.max()) <= cap


def test_cache_checkpoint_restore_is_bit_exact(gpu_lib):
    """The decode state is the caller's tensors: copying them out, running on,
    restoring and re-running gives bit-identical outputs."""
    cfg, N0, seed = DEC_CASES["bf16_G4"]
    raw = workloads.make_prefill(cfg, seed)
    dev, _ = prepare(raw, torch.bfloat16)
    gc = gpu_lib.DecodeCache(batch=2, n_kv_heads=2, head_dim=128, window=64, chunk=64, topk=16,
                             sel_cap=128, pos=N0)
    gpu_lib.fwd(dev["q"][:, :N0].contiguous(), dev["k"][:, :N0].contiguous(),
                dev["v"][:, :N0].contiguous(), dev["wphi_q"], dev["wphi_k"], window=64, chunk=64,
                topk=16, cache=gc)
    snap = {k: v.clone() for k, v in gc.tensors().items()}

    def run():
        outs = []
        for t in range(N0, N0 + 70):
            outs.append(gpu_lib.decode_step(dev["q"][:, t:t + 1].contiguous(),
                                            dev["k"][:, t:t + 1].contiguous(),
                                            dev["v"][:, t:t + 1].contiguous(), dev["wphi_q"],
                                            dev["wphi_k"], gc).clone())
        return torch.cat(outs, 1)

    a = run()
    for k, v in snap.items():
        getattr(gc, k).copy_(v)
    gc.pos = N0
    b = run()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ragged batches: each sequence at its own position (serving form of the step)
RAGGED_CASES = {
    # name: (cfg with seqlen = max(N0) + steps, per-sequence N0, steps, seed)
    "bf16_G4": (make_case("r", 3, 191 + 70, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0),
                [70, 130, 191], 70, 51),
    "f32_W32_C16": (make_case("s", 3, 77 + 40, 4, 1, 64, 32, 16, 4, dtype="f32"), [0, 40, 77], 40, 52),
}


def cache_slice(gc, b):
    """A batch-1 view of sequence b of a DecodeCache (same memory)."""
    sl = copy.copy(gc)
    for key in ("win_k", "win_v", "win_route", "pend_score", "sel_k", "sel_v", "sel_count", "lin_S",
                "lin_z"):
        setattr(sl, key, getattr(gc, key)[b:b + 1])
    sl._struct = None
    return sl


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(RAGGED_CASES))
def test_ragged_positions_decode(gpu_lib, name, general):
    """Sequences prefilled to different lengths (each by its own forward into
    its slice of one cache), then decoded together with one position per
    sequence: every step's output and the final caches match the oracle's
    recurrent form run per sequence, and the positions advance on the GPU."""
    cfg, n0s, steps, seed = RAGGED_CASES[name]
    say(f"[ragged] case={name} general={general} shape={workloads.shape_of(cfg)} N0={n0s} "
        f"steps={steps} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    B = cfg["batch"]
    Hkv, d = cfg["n_kv_heads"], cfg["head_dim"]
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    p = O.Params(window=W, chunk=C, topk=lam)
    cap = p.topk_eff() * (-(-cfg["seqlen"] // C)) + 1
    tol = F32_TOL if cfg["dtype"] == "f32" else BF16_TOL
    one = dict(cfg, batch=1)

    gc = gpu_lib.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C, topk=lam,
                             sel_cap=cap, dtype=dt)
    ocs = []
    for b, n0 in enumerate(n0s):
        sl = cache_slice(gc, b)
        sl.pos = n0
        if n0 > 0:
            gpu_lib.fwd(dev["q"][b:b + 1, :n0].contiguous(), dev["k"][b:b + 1, :n0].contiguous(),
                        dev["v"][b:b + 1, :n0].contiguous(), dev["wphi_q"], dev["wphi_k"], window=W,
                        chunk=C, topk=lam, cache=sl, general=general)
        _, oc = O.fwd_recurrent(ref["q"][b:b + 1, :n0], ref["k"][b:b + 1, :n0], ref["v"][b:b + 1, :n0],
                                ref["wphi_q"], ref["wphi_k"], p, cap=cap)
        ocs.append(oc)
    torch.cuda.synchronize()
    pos = torch.tensor(n0s, dtype=torch.int64, device="cuda")
    worst = 0.0
    for s in range(steps):
        idx = [n0 + s for n0 in n0s]
        q_t = torch.stack([dev["q"][b, t] for b, t in enumerate(idx)])[:, None].contiguous()
        k_t = torch.stack([dev["k"][b, t] for b, t in enumerate(idx)])[:, None].contiguous()
        v_t = torch.stack([dev["v"][b, t] for b, t in enumerate(idx)])[:, None].contiguous()
        g_out = gpu_lib.decode_step_ragged(q_t, k_t, v_t, dev["wphi_q"], dev["wphi_k"], gc, pos,
                                           max(idx), general=general)
        torch.cuda.synchronize()
        g = g_out[:, 0].double().cpu().numpy()
        for b, t in enumerate(idx):
            o_out = O.decode_step(ocs[b], ref["q"][b:b + 1, t], ref["k"][b:b + 1, t],
                                  ref["v"][b:b + 1, t], ref["wphi_q"], ref["wphi_k"], p)
            err = rel_l2(g[b:b + 1], o_out)
            worst = max(worst, err)
            assert err <= tol, f"sequence {b} step t={t}: rel-L2 {err:.3e}"
            check_rows(g[b:b + 1], o_out, row_tol(cfg["dtype"]), what=f"sequence {b} step t={t}")
    assert pos.cpu().tolist() == [n0 + steps for n0 in n0s]
    for b, n0 in enumerate(n0s):
        compare_cache(cache_slice(gc, b), ocs[b], one, n0 + steps, 1e-5)
    say(f"  {steps} ragged steps, worst rel-L2 {worst:.3e}; caches match")


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("route", ["diagonal", "qk", "keynorm", "uniform", "random"])
def test_decode_routing_criteria(gpu_lib, route, general):
    """Hand-off and decode steps under each routing criterion: the chunk-end
    decisions of the recurrent form use the criterion's pending scores."""
    cfg = make_case("j", 2, 130 + 70, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0)
    N0, seed = 130, 61
    say(f"[decode route] {route} general={general} shape={workloads.shape_of(cfg)} N0={N0}")
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch.bfloat16)
    B, N, Hkv, d = cfg["batch"], cfg["seqlen"], cfg["n_kv_heads"], cfg["head_dim"]
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    p = O.Params(window=W, chunk=C, topk=lam, route=route)
    cap = p.topk_eff() * (-(-N // C)) + 1
    gc = gpu_lib.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C, topk=lam,
                             sel_cap=cap, pos=N0)
    gpu_lib.fwd(dev["q"][:, :N0].contiguous(), dev["k"][:, :N0].contiguous(), dev["v"][:, :N0].contiguous(),
                dev["wphi_q"], dev["wphi_k"], window=W, chunk=C, topk=lam, cache=gc, general=general,
                route=route)
    _, oc = O.fwd_recurrent(ref["q"][:, :N0], ref["k"][:, :N0], ref["v"][:, :N0], ref["wphi_q"],
                            ref["wphi_k"], p, cap=cap)
    torch.cuda.synchronize()
    compare_cache(gc, oc, cfg, N0, 1e-5)
    worst = 0.0
    for t in range(N0, N):
        g_out = gpu_lib.decode_step(dev["q"][:, t:t + 1].contiguous(), dev["k"][:, t:t + 1].contiguous(),
                                    dev["v"][:, t:t + 1].contiguous(), dev["wphi_q"], dev["wphi_k"], gc,
                                    general=general, route=route)
        o_out = O.decode_step(oc, ref["q"][:, t], ref["k"][:, t], ref["v"][:, t], ref["wphi_q"],
                              ref["wphi_k"], p)
        torch.cuda.synchronize()
        g_np = g_out[:, 0].double().cpu().numpy()
        err = rel_l2(g_np, o_out)
        worst = max(worst, err)
        assert err <= BF16_TOL, f"step t={t}: rel-L2 {err:.3e}"
        check_rows(g_np, o_out, row_tol("bf16"), what=f"step t={t}")
    compare_cache(gc, oc, cfg, N, 1e-5)
    say(f"  {N - N0} steps, worst rel-L2 {worst:.3e}")
