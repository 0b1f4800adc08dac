"""GPU parity of the backward pass (gradients of sum(dout * out) w.r.t. q,
k, v and both NP-Map projections, routing held fixed) against the float64
oracle's bwd_direct, whole tensors, at sizes the oracle finishes in seconds
(several chunks and a ragged tail), plus the method's degenerate cases and a
property check at the 4K prefill size.

The routing differentiated under is the GPU forward's own selection, handed
to both sides, so selection near-ties cannot matter here.  Bar: rel-L2 of
every gradient tensor <= 1e-4.  The gradients are fp32 sums of fp32 terms
from the same (dtype-rounded) inputs the oracle gets in float64; the longest
sums have a few thousand terms, whose rounding stays near 1e-6 relative, so
1e-4 leaves two orders of magnitude of room while a wrong term, sign or
index shows up at 1e-2 or more.

The matrix-core path (bf16 storage, d = 128, chunk 64 / 128 / 256 up to the
window 64 / 128 / 256, 1 / 2 / 4 / 8 query heads per KV head) takes the statistics from the
forward's bf16 pass (probabilities rounded to bf16), rounds dS and P to bf16
before their products, and runs the linear terms (bf16 prefix states,
features and chunk sums), the NP-Map backward (bf16 P^T and du) and the
projection gradients (bf16 du) on the matrix cores too, so its gradients
carry bf16 operand rounding (2^-9 relative per term): its bar is
MFMA_GRAD_TOL per tensor, and every case also runs on the fp32 general
kernels at 1e-4."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import check_rows, make_case, prepare, rel_l2, say, torch_dtype

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-4
MFMA_GRAD_TOL = 2e-2


def mfma_path(cfg) -> bool:
    """Whether the library takes the matrix-core backward for this shape."""
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    return (cfg["dtype"] == "bf16" and cfg["head_dim"] == 128 and cfg["chunk"] in (64, 128, 256)
            and cfg["window"] in (64, 128, 256) and cfg["window"] >= cfg["chunk"] and G in (1, 2, 4, 8))


# Anti-aligned inputs (every key -a u plus noise, a = 56 against a spread of
# about 11) make dq = tau sum_j dS_j k_j cancel the keys' common part, which
# amplifies the bf16 rounding of dS by |k| / |k - mean k|, about 5.
MFMA_GRAD_TOL_ANTI_ALIGNED = 5 * MFMA_GRAD_TOL


def grad_tol(cfg, general) -> float:
    if not mfma_path(cfg) or general:
        return GRAD_TOL
    return MFMA_GRAD_TOL_ANTI_ALIGNED if cfg.get("anti_align") else MFMA_GRAD_TOL
NAMES = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dwphi_q", "dwq"), ("dwphi_k", "dwk"))

CASES = {
    "bf16_ragged_G2": (make_case("r", 1, 300, 4, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 31),
    "f32_d64_W32_C32": (make_case("a", 2, 200, 2, 1, 64, 32, 32, 8, dtype="f32"), 32),
    "f32_W_gt_C_G8": (make_case("b", 1, 150, 8, 1, 64, 48, 16, 4, dtype="f32"), 33),
    "bf16_swa_la": (make_case("c", 1, 230, 4, 2, 128, 64, 64, 0), 34),
    "f32_pure_linear": (make_case("d", 1, 130, 2, 1, 64, 0, 32, 0, dtype="f32"), 35),
    "bf16_all_selected": (make_case("e", 1, 200, 4, 2, 128, 64, 64, 64), 36),
    "bf16_short_no_chunk": (make_case("f", 2, 40, 4, 2, 128, 64, 64, 16), 37),
    "bf16_single_token": (make_case("g", 1, 1, 4, 2, 128, 64, 64, 16), 38),
    # one query head per KV head, and the Llama 32 / 8 grouping (four per KV
    # head) with linear tokens present, so the projection gradients are not 0
    "bf16_G1": (make_case("h", 1, 300, 2, 2, 128, 64, 64, 16), 39),
    "bf16_G4_linear": (make_case("i", 1, 300, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 40),
    # three query heads per KV head: the padded heads of the grouped kernels
    "f32_G3_d64": (make_case("j", 1, 200, 6, 2, 64, 32, 32, 8, dtype="f32"), 41),
    # fp32 storage at d = 128
    "f32_d128_G2": (make_case("k", 1, 200, 4, 2, 128, 64, 64, 16, dtype="f32"), 42),
    # every logit far below -100 (queries along +56 u, keys along -56 u):
    # queries with no linear term must keep finite softmax statistics
    "bf16_underflow_all_selected": (make_case("u", 1, 200, 4, 2, 128, 64, 64, 64, anti_align=56.0), 43),
    "bf16_underflow_G2": (make_case("v", 1, 300, 4, 2, 128, 64, 64, 16, anti_align=56.0), 44),
    # windows of two and four chunks (W = 128 / 256, C = 64)
    "bf16_W128_C64_G4": (make_case("w", 1, 450, 8, 2, 128, 128, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 46),
    "bf16_W256_C64_G2": (make_case("x", 1, 600, 4, 2, 128, 256, 64, 8), 47),
    # chunks of 128 / 256 tokens (the chunk-size ablation, W >= C): selection
    # per chunk, the matrix-core kernels in 64-token tiles; lam > 64 puts up
    # to 64 selected rows in one tile
    "bf16_W128_C128_G4": (make_case("y", 1, 400, 8, 2, 128, 128, 128, 16, outlier_frac=0.02, heavy_scale=6.0), 48),
    "bf16_W256_C128_G2": (make_case("z", 1, 600, 4, 2, 128, 256, 128, 40), 49),
    "bf16_W256_C256_G1_lam100": (make_case("z", 1, 700, 2, 2, 128, 256, 256, 100), 50),
    "bf16_W128_C128_swa_la": (make_case("z", 1, 350, 4, 1, 128, 128, 128, 0), 51),
    # eight query heads per KV head: the query-side kernel's blocks take four
    # heads each, so two blocks share every (KV head, chunk)
    "bf16_G8": (make_case("l", 1, 300, 16, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 52),
    "bf16_W128_C128_G8": (make_case("m", 1, 330, 8, 1, 128, 128, 128, 24), 53),
    # wide chunks at the ends of the routing: every token selected (each
    # 64-token tile of the lists full), and no selection (window + linear)
    "bf16_W128_C128_all_selected": (make_case("n", 1, 400, 4, 2, 128, 128, 128, 128), 54),
    "bf16_W256_C256_swa_la": (make_case("p", 1, 700, 4, 2, 128, 256, 256, 0), 55),
}


def run(gpu_lib, cfg, seed, corrupt=False, general=False, saved=False, fwd_general=False, fwd_ws=False):
    """saved: the backward starts from the forward's out and statistics (the
    forward on the general kernels when fwd_general); fwd_ws: and from the
    forward's workspace (its keys' features and linear prefixes)."""
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(dt)
    ref_dout = dout.double().numpy()
    dout = dout.cuda().contiguous()
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    sel = None
    fw = None
    if min(lam, C) > 0 or saved:
        fw = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W,
                         chunk=C, topk=lam, return_sel=min(lam, C) > 0, return_stats=saved,
                         general=fwd_general, return_workspace=fwd_ws)
        sel = fw.get("sel_idx")
    osel = None if sel is None else sel.cpu().numpy().astype(np.int64)
    if corrupt and sel is not None and sel.shape[2] > 1:
        # a repeated entry and an out-of-chunk entry are ignored by the library;
        # the oracle gets the same routing with the bad entry as a repeat
        bad = sel.clone()
        bad[:, :, 0, 1] = bad[:, :, 0, 0]
        bad[:, :, 1, 0] = 1 << 30
        osel = bad.cpu().numpy().astype(np.int64)
        osel[:, :, 1, 0] = osel[:, :, 1, 1]
        sel = bad
    extra = dict(out=fw["out"], stats=fw["stats"]) if saved else {}
    if fwd_ws:
        extra["fwd_workspace"] = fw["workspace"]
    g = gpu_lib.bwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], sel, dout,
                    window=W, chunk=C, topk=lam, general=general, **extra)
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam)
    o = O.bwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], ref_dout, p,
                     sel_idx=osel)
    return g, o


def compare(g, o, tol=GRAD_TOL):
    errs = {}
    for gname, oname in NAMES:
        x = g[gname].double().cpu().numpy()
        assert np.isfinite(x).all(), gname
        errs[gname] = rel_l2(x, o[oname]) if np.any(o[oname]) else float(np.abs(x).max())
    say("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(CASES))
def test_bwd_matches_oracle(gpu_lib, name, general):
    cfg, seed = CASES[name]
    say(f"[bwd] case={name} general={general} matrix-core={mfma_path(cfg) and not general} "
        f"shape={workloads.shape_of(cfg)} seed={seed}")
    g, o = run(gpu_lib, cfg, seed, general=general)
    compare(g, o, grad_tol(cfg, general))


SAVED_CASES = ["bf16_ragged_G2", "bf16_G1", "bf16_G4_linear", "bf16_swa_la", "bf16_all_selected",
               "bf16_short_no_chunk", "bf16_single_token", "bf16_underflow_G2", "bf16_underflow_all_selected",
               "bf16_W128_C64_G4", "bf16_W256_C64_G2", "bf16_W128_C128_G4", "bf16_W256_C256_G1_lam100",
               "bf16_G8", "f32_d128_G2"]


@pytest.mark.parametrize("fwd", ["picked", "picked_ws", "general"], ids=lambda x: "fwd_" + x)
@pytest.mark.parametrize("name", SAVED_CASES)
def test_bwd_from_forward_statistics_matches_oracle(gpu_lib, name, fwd):
    """The backward started from the forward's out and statistics (no first
    pass on the matrix cores) against the oracle, with the statistics from
    either forward path: both define (m, l) at their own reference point, so
    either must do.  picked_ws: the backward also takes the keys' features
    and linear prefixes from the matrix-core forward's workspace.  The fp32
    kernels ignore both."""
    cfg, seed = CASES[name]
    fwd_general = fwd == "general"
    say(f"[bwd] from forward stats case={name} fwd={fwd} "
        f"matrix-core={mfma_path(cfg)} shape={workloads.shape_of(cfg)} seed={seed}")
    g, o = run(gpu_lib, cfg, seed, saved=True, fwd_general=fwd_general, fwd_ws=fwd == "picked_ws")
    compare(g, o, grad_tol(cfg, False))


@pytest.mark.parametrize("name", ["bf16_G4_linear", "bf16_W256_C64_G2", "bf16_W128_C128_G8"])
def test_bwd_forward_workspace_gives_the_recomputed_linear_state(gpu_lib, name):
    """The linear state the backward reads from the forward's workspace is
    the one it would recompute (same kernels, same routing): the gradients
    with and without the workspace agree to fp32 rounding, so the handed-over
    buffers line up with the backward's own."""
    cfg, seed = CASES[name]
    say(f"[bwd] forward workspace vs recomputed linear state case={name} shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, _ = prepare(raw, dt)
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(dt).cuda().contiguous()
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    args = (dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"])
    fw = gpu_lib.fwd(*args, window=W, chunk=C, topk=lam, return_sel=True, return_stats=True,
                     return_workspace=True)
    saved = dict(out=fw["out"], stats=fw["stats"])
    a = gpu_lib.bwd(*args, fw["sel_idx"], dout, window=W, chunk=C, topk=lam, **saved)
    b = gpu_lib.bwd(*args, fw["sel_idx"], dout, window=W, chunk=C, topk=lam, **saved,
                    fwd_workspace=fw["workspace"])
    torch.cuda.synchronize()
    for gname, _ in NAMES:
        x, y = a[gname].double().cpu().numpy(), b[gname].double().cpu().numpy()
        err = np.abs(x - y).max() / max(np.abs(x).max(), 1e-30)
        say(f"  {gname} max difference / max {err:.2e}")
        assert np.isfinite(y).all() and err <= 1e-6, (gname, err)


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", ["bf16_ragged_G2", "bf16_W128_C128_G4"])
def test_bwd_ignores_repeated_and_foreign_selection_entries(gpu_lib, name, general):
    cfg, seed = CASES[name]
    say(f"[bwd] corrupted selection general={general} shape={workloads.shape_of(cfg)} seed={seed}")
    g, o = run(gpu_lib, cfg, seed, corrupt=True, general=general)
    compare(g, o, grad_tol(cfg, general))


def test_bwd_is_deterministic(gpu_lib):
    cfg, seed = CASES["bf16_ragged_G2"]
    raw = workloads.make_prefill(cfg, seed)
    dev, _ = prepare(raw, torch.bfloat16)
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(torch.bfloat16).cuda()
    sel = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=64,
                      chunk=64, topk=16, return_sel=True)["sel_idx"]
    runs = [gpu_lib.bwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], sel, dout,
                        window=64, chunk=64, topk=16) for _ in range(2)]
    torch.cuda.synchronize()
    for key in runs[0]:
        assert torch.equal(runs[0][key], runs[1][key]), key


def test_bwd_empty_sequence_zeroes_projection_gradients(gpu_lib):
    q = torch.zeros((1, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, 64, 128), dtype=torch.float32, device="cuda")
    g = gpu_lib.bwd(q, k, k, w, w, None, q, window=64, chunk=64, topk=16)
    torch.cuda.synchronize()
    assert g["dq"].shape == (1, 0, 4, 128)
    assert torch.count_nonzero(g["dwphi_q"]) == 0 and torch.count_nonzero(g["dwphi_k"]) == 0


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
def test_bwd_all_selected_at_4k_is_causal_softmax_gradient(gpu_lib, general):
    """At the 4K prefill shape (32 / 8 heads, d 128) with every routed token
    selected (topk = C) the operator is causal softmax attention, a property
    that holds at any size: its gradients must be those of torch's SDPA
    (float32 autograd on the GPU) and the projections get none."""
    cfg = dict(workloads.CONFIGS["prefill_4k"], topk=64)
    seed = workloads.seed_of("prefill_4k")
    say(f"[bwd] 4k all-selected general={general} shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dev, _ = prepare(raw, torch.bfloat16)
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(torch.bfloat16).cuda()
    sel = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=64,
                      chunk=64, topk=64, return_sel=True)["sel_idx"]
    g = gpu_lib.bwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], sel, dout,
                    window=64, chunk=64, topk=64, general=general)
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    tq = dev["q"].float().permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = dev["k"].float().permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = dev["v"].float().permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), is_causal=True)
    (o * dout.float().permute(0, 2, 1, 3)).sum().backward()
    torch.cuda.synchronize()
    ref = {"dq": tq.grad.permute(0, 2, 1, 3), "dk": tk.grad.permute(0, 2, 1, 3),
           "dv": tv.grad.permute(0, 2, 1, 3)}
    for key, r in ref.items():
        err = rel_l2(g[key].double().cpu().numpy(), r.double().cpu().numpy())
        say(f"  {key} rel-L2 vs SDPA {err:.2e}")
        assert err <= grad_tol(cfg, general)
    assert torch.count_nonzero(g["dwphi_q"]) == 0 and torch.count_nonzero(g["dwphi_k"]) == 0


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
def test_bwd_train_8x2k_sampled_rows_and_value_sums(gpu_lib, general):
    """At the full training-batch size (8 x 2048, 32 / 8 heads, d 128, top-16)
    in the bench's launch configuration: dq on sampled query rows against the
    oracle, one row at a time; and sum_j dv_j = the sum of dout over the
    group's queries, because every query's weights over its softmax and
    linear tokens sum to one -- a property of the whole routing at any size,
    held to the fp32 rounding of the sums (1e-5 of sum_j |dv_j|), or on the
    matrix-core path to the bf16 rounding of the first pass's probabilities
    (their sum l, and so each query's weights, carry 2^-9 relative rounding:
    4e-3 of sum_j |dv_j|)."""
    from parity import sampled_rows
    name = "train_8x2k"
    cfg, seed = workloads.CONFIGS[name], workloads.seed_of(name)
    say(f"[bwd] {name} sampled rows general={general} shape={workloads.shape_of(cfg)} seed={seed}")
    tol = grad_tol(cfg, general)
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch.bfloat16)
    dout_h = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(torch.bfloat16)
    dout = dout_h.cuda()
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    sel = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                      topk=lam, return_sel=True)["sel_idx"]
    g = gpu_lib.bwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], sel, dout,
                    window=W, chunk=C, topk=lam, general=general)
    torch.cuda.synchronize()
    B, N, Hq, d = dev["q"].shape
    Hkv = cfg["n_kv_heads"]
    rows = sampled_rows(B, N, C, n_per_batch=3, seed=5)
    p = O.Params(window=W, chunk=C, topk=lam)
    o = O.bwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"],
                     dout_h.double().numpy(), p, sel_idx=sel.cpu().numpy().astype(np.int64), rows=rows)
    bi, ti = np.array([r[0] for r in rows]), np.array([r[1] for r in rows])
    err = rel_l2(g["dq"].double().cpu().numpy()[bi, ti], o["dq"][bi, ti])
    say(f"  dq rel-L2 over {len(rows)} sampled rows: {err:.2e}")
    assert err <= tol
    # key side on sampled keys of one sequence and KV head: selected keys,
    # linear keys, keys still in the window at the end, the last chunk's keys
    b0, g0 = 3, 5
    sel_np = sel.cpu().numpy().astype(np.int64)
    picked = sorted(set(sel_np[b0, g0].reshape(-1).tolist()))
    linear = [j for j in range(0, N - W) if j not in set(picked)]
    rng = np.random.default_rng(7)
    js = set(rng.choice(picked, 6, replace=False).tolist()) | set(rng.choice(linear, 6, replace=False).tolist())
    js |= {0, 1, C - 1, N - W - 1, N - W, N - C, N - 2, N - 1} | {picked[-1], linear[-1]}
    keys = [(b0, g0, j) for j in sorted(js)]
    ok = O.bwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"],
                      dout_h.double().numpy(), p, sel_idx=sel_np, keys=keys)
    jj = np.array(sorted(js))
    for gname in ("dk", "dv"):
        got = g[gname].double().cpu().numpy()[b0, jj, g0]
        want = ok[gname][b0, jj, g0]
        err = rel_l2(got, want)
        say(f"  {gname} rel-L2 over {len(jj)} sampled keys of (b={b0}, g={g0}): {err:.2e}")
        assert err <= tol
        check_rows(got, want, 10 * tol, what=gname)
    dv = g["dv"].double()
    lhs = dv.sum(dim=1)                                           # [B, Hkv, d]
    rhs = dout_h.double().cuda().reshape(B, N, Hkv, Hq // Hkv, d).sum(dim=(1, 3))
    bound = (4e-3 if tol > GRAD_TOL else 1e-5) * dv.abs().sum(dim=1) + 1e-6
    worst = float(((lhs - rhs).abs() / bound).max())
    say(f"  sum_j dv_j vs sum of dout: worst |diff| / bound {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("chunk", [64, 128])
def test_bwd_projection_gradients_mid_size(gpu_lib, chunk):
    """The NP-Map projection gradients, which sum over every token of every
    head of a KV group, at a mid size (1 x 1024, 8 / 2 heads, d 128, top-16,
    W = C = 64 or 128): whole tensors against the oracle, with dq, dk and dv."""
    cfg = make_case("m", 1, 1024, 8, 2, 128, chunk, chunk, 16, outlier_frac=0.01, heavy_scale=6.0)
    seed = 45
    for general in (False, True):
        say(f"[bwd] mid-size projections general={general} shape={workloads.shape_of(cfg)} seed={seed}")
        g, o = run(gpu_lib, cfg, seed, general=general)
        compare(g, o, grad_tol(cfg, general))
