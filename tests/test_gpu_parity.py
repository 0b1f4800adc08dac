"""GPU parity of the chunk-parallel forward against the float64 oracle, whole
tensors, element by element, at sizes the oracle finishes in seconds (several
tiles and a ragged tail), plus the method's degenerate cases.

Bars: selected positions bit-exact (or the near-tie protocol), output rel-L2
<= 1e-2 for bf16 storage and <= 1e-5 for fp32, group scores within 1e-4
relative.  Every case runs through the C ABI, both with the kernels the
library picks for the shape and with the general kernels forced."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import (BF16_TOL, F32_TOL, check_rows, check_selection, make_case, prepare, rel_l2,
                    row_tol, say, torch_dtype)

pytestmark = pytest.mark.gpu

CASES = {
    "toy_fp32": (workloads.CONFIGS["toy_fp32"], workloads.seed_of("toy_fp32")),
    "bf16_ragged_G4": (make_case("r", 2, 600, 8, 2, 128, 64, 64, 16, outlier_frac=0.01, heavy_scale=6.0), 11),
    "bf16_tiles_G4": (make_case("t", 1, 1024, 8, 2, 128, 64, 64, 32, outlier_frac=0.01, heavy_scale=6.0), 12),
    "bf16_d64_W96_C32": (make_case("a", 1, 333, 4, 1, 64, 96, 32, 8), 13),
    "f32_G8_d64": (make_case("b", 1, 200, 8, 1, 64, 32, 16, 5, dtype="f32"), 14),
    "bf16_all_selected": (make_case("c", 1, 300, 4, 2, 128, 64, 64, 64), 15),
    "bf16_window_covers": (make_case("d", 1, 200, 4, 2, 128, 256, 64, 0), 16),
    "bf16_pure_linear": (make_case("e", 1, 200, 4, 2, 128, 0, 64, 0), 17),
    "bf16_short_no_chunk": (make_case("f", 2, 50, 4, 2, 128, 64, 64, 16), 18),
    "bf16_G1": (make_case("g", 1, 400, 2, 2, 128, 64, 64, 16), 19),
    "bf16_G8": (make_case("h", 1, 320, 8, 1, 128, 64, 64, 8), 20),
    "f32_lam_gt_C": (make_case("i", 1, 256, 4, 1, 64, 32, 32, 40, dtype="f32"), 21),
    "bf16_swa_la_W_lt_C": (make_case("j", 1, 300, 4, 1, 128, 40, 64, 0), 22),
    # SWA + linear (no selection) at W = C = 64: the matrix-core path with no
    # compact rows, every routed token linear
    "bf16_swa_la_W_eq_C": (make_case("l", 2, 333, 8, 2, 128, 64, 64, 0, outlier_frac=0.01, heavy_scale=6.0), 31),
    # window of two chunks (W = 128, C = 64: the pages' full-RULER window):
    # the matrix-core path with the window spanning chunks c-2 .. c
    "bf16_W128_C64_G4": (make_case("m", 2, 700, 8, 2, 128, 128, 64, 16, outlier_frac=0.01, heavy_scale=6.0), 32),
    "bf16_W128_C64_G1": (make_case("n", 1, 450, 2, 2, 128, 128, 64, 8), 33),
    "bf16_W128_C64_G8_swa_la": (make_case("o", 1, 400, 8, 1, 128, 128, 64, 0), 34),
    "bf16_W128_C64_all_selected": (make_case("p", 1, 333, 4, 2, 128, 128, 64, 64), 35),
    "bf16_W128_C64_underflow": (make_case("q", 1, 350, 8, 2, 128, 128, 64, 16, anti_align=56.0), 36),
    # four-chunk window (W = 256, C = 64: the widest S-NIAH window)
    "bf16_W256_C64_G4": (make_case("r", 2, 700, 8, 2, 128, 256, 64, 16, outlier_frac=0.01, heavy_scale=6.0), 37),
    "bf16_W256_C64_G2_swa_la": (make_case("s", 1, 500, 4, 2, 128, 256, 64, 0), 38),
    # chunks of 128 and 256 tokens (the pages' chunk-size ablation runs W = C;
    # W = 256 over C = 128 as well): the matrix-core path selects per chunk and
    # runs everything after the selection in 64-token tiles.  Ragged tails end
    # inside the open chunk; "lam_gt_64" ends on a complete chunk.
    "bf16_W128_C128_G4": (make_case("z", 2, 700, 8, 2, 128, 128, 128, 16, outlier_frac=0.01, heavy_scale=6.0), 40),
    "bf16_W256_C128_G2": (make_case("z", 1, 900, 4, 2, 128, 256, 128, 32), 41),
    "bf16_W256_C256_G8": (make_case("z", 1, 1100, 8, 1, 128, 256, 256, 48, outlier_frac=0.01, heavy_scale=6.0), 42),
    "bf16_W128_C128_lam_gt_64": (make_case("z", 1, 640, 4, 2, 128, 128, 128, 100), 43),
    "bf16_W128_C128_swa_la": (make_case("z", 1, 500, 4, 1, 128, 128, 128, 0), 44),
    "bf16_W128_C128_underflow": (make_case("z", 1, 400, 8, 2, 128, 128, 128, 16, anti_align=56.0), 45),
    # matrix-core path with two query heads per KV head, three sequences, a ragged tail
    "bf16_G2_B3_ragged": (make_case("k", 3, 777, 4, 2, 128, 64, 64, 20, outlier_frac=0.02, heavy_scale=6.0), 23),
    # keys scaled x80 at 2% of positions: logits beyond 2^128 in exp2 units, so
    # the matrix-core path's fixed-reference pass overflows and its second
    # pass (running reference) recomputes those blocks
    "bf16_overflow_G4": (make_case("o", 1, 700, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=80.0), 24),
    # queries along +56 u and keys along -56 u: every logit lies far below -100
    # (natural units), below fp32's exp range.  Queries with no linear term
    # (the first chunks; every query when every routed token is selected, or
    # when the window covers the sequence) must keep their softmax finite.
    "bf16_underflow_all_selected": (make_case("u", 1, 333, 8, 2, 128, 64, 64, 64, anti_align=56.0), 26),
    "bf16_underflow_G4": (make_case("v", 2, 300, 8, 2, 128, 64, 64, 16, anti_align=56.0), 27),
    "bf16_underflow_G2": (make_case("w", 1, 260, 4, 2, 128, 64, 64, 16, anti_align=56.0), 28),
    "bf16_underflow_window_covers": (make_case("x", 1, 150, 4, 2, 128, 256, 64, 0, anti_align=56.0), 29),
    "f32_underflow_d64": (make_case("y", 1, 200, 4, 1, 64, 32, 16, 16, dtype="f32", anti_align=48.0), 30),
}
OVERFLOW_CASES = {"bf16_overflow_G4"}
UNDERFLOW_CASES = {n for n in CASES if "underflow" in n}


def largest_causal_logit(cfg, seed):
    """max over heads and causal pairs of tau q.k, natural units, on the
    dtype-rounded inputs."""
    _, ref = prepare(workloads.make_prefill(cfg, seed), torch_dtype(cfg["dtype"]), device="cpu")
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    n = cfg["seqlen"]
    causal = np.tril(np.ones((n, n), dtype=bool))
    top = max(float(np.max(np.where(causal, ref["q"][b, :, h] @ ref["k"][b, :, h // G].T, -np.inf)))
              for b in range(cfg["batch"]) for h in range(cfg["n_q_heads"]))
    return top / np.sqrt(cfg["head_dim"])


def run_case(gpu_lib, cfg, seed, general):
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, ref = prepare(raw, dt)
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W,
                      chunk=C, topk=lam, return_scores=True, return_sel=True, general=general)
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam)
    Hkv = cfg["n_kv_heads"]
    sigma = O.window_scores(ref["q"], ref["k"], p, Hkv) if W > 0 else np.zeros(
        (cfg["batch"], Hkv, cfg["seqlen"]))
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    override = None
    if p.topk_eff() > 0:
        osel, _ = O.select_chunks(sigma, p)
        n_bad, worst = check_selection(gsel, sigma, osel, C)
        if n_bad:
            say(f"  near-tie chunks: {n_bad} (worst margin {worst:.3g}); oracle re-run with GPU picks")
            override = gsel
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p,
                     sel_override=override, scores=sigma)
    return res, o, sigma


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", list(CASES))
def test_fwd_matches_oracle(gpu_lib, name, general):
    cfg, seed = CASES[name]
    say(f"[fwd] case={name} general={general} shape={workloads.shape_of(cfg)} seed={seed}")
    res, o, sigma = run_case(gpu_lib, cfg, seed, general)
    out = res["out"].double().cpu().numpy()
    assert np.isfinite(out).all()
    err = rel_l2(out, o["out"])
    tol = F32_TOL if cfg["dtype"] == "f32" else BF16_TOL
    if cfg["window"] > 0:
        gs = res["scores"].cpu().numpy()
        serr = float(np.max(np.abs(gs - sigma) / np.maximum(1.0, np.abs(sigma))))
    else:
        serr = 0.0
    if name in OVERFLOW_CASES:
        # the case must reach logits whose exp2 overflows fp32 (> 128 in log2 units)
        top = largest_causal_logit(cfg, seed) * np.log2(np.e)
        say(f"  largest causal logit {top:.1f} (log2 units)")
        assert top > 130.0
    if name in UNDERFLOW_CASES:
        # every logit must lie below -100 (natural units): exp underflows in fp32
        top = largest_causal_logit(cfg, seed)
        say(f"  largest causal logit {top:.1f} (natural units)")
        assert top < -100.0
    say(f"  out rel-L2 {err:.3e} (tol {tol:g}), score max rel err {serr:.3e}")
    assert err <= tol
    check_rows(out, o["out"], row_tol(cfg["dtype"]))
    assert serr <= 1e-4


STATS_CASES = ["bf16_ragged_G4", "bf16_G1", "bf16_G8", "bf16_swa_la_W_eq_C", "bf16_all_selected",
               "bf16_window_covers", "bf16_pure_linear", "bf16_overflow_G4", "bf16_underflow_G4",
               "bf16_W128_C64_G4", "bf16_W128_C128_G4", "toy_fp32", "f32_G8_d64"]


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("name", STATS_CASES)
def test_fwd_statistics_match_oracle(gpu_lib, name, general):
    """The statistics the forward hands a backward, (m, l, 0, c) per query
    head: m + ln l is the log of the shared normaliser whatever the reference
    m (list view Fig. 2), c = exp(-m) / l exactly for the queries with linear
    weight and 0 for the others."""
    cfg, seed = CASES[name]
    say(f"[fwd stats] case={name} general={general} shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch_dtype(cfg["dtype"]))
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                      topk=lam, return_sel=True, return_stats=True, general=general)
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam)
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64) if p.topk_eff() > 0 else None
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p, sel_override=gsel)
    st = res["stats"].double().cpu().numpy()
    m, l, zero, c = st[..., 0], st[..., 1], st[..., 2], st[..., 3]
    assert np.isfinite(st).all() and (l > 0).all() and (zero == 0).all()
    err = float(np.max(np.abs(m + np.log(l) - o["lse"])))
    tol = 1e-5 if cfg["dtype"] == "f32" else 1e-2
    say(f"  max |m + ln l - lse| {err:.2e} (tol {tol:g})")
    assert err <= tol
    lin = o["has_linear"]
    assert (c[~lin] == 0).all()
    # where exp(-lse) is a normal fp32 number (not under the keys x80 outliers)
    ok = lin & (o["lse"] < 80.0)
    if ok.any():
        cerr = float(np.max(np.abs(c[ok] * np.exp(o["lse"][ok]) - 1.0)))
        say(f"  max |c exp(lse) - 1| over {int(ok.sum())} rows with linear weight {cerr:.2e}")
        assert cerr <= tol


@pytest.mark.parametrize("W,C", [(64, 64), (128, 64), (128, 128), (256, 128), (256, 256)])
def test_matrix_core_path_taken(gpu_lib, W, C):
    """The pages' (W, C) settings with d = 128 in bf16 run on the matrix-core
    kernels: the timed entry point names the launches it made."""
    cfg = make_case("p", 1, 300, 4, 2, 128, W, C, 16)
    dev, _ = prepare(workloads.make_prefill(cfg, 50), torch.bfloat16)
    timer = gpu_lib.LaunchTimer()
    gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C, topk=16,
                timer=timer)
    names = [n for n, _ in timer.durations_ms()]
    want = ["win_select"] + (["chunk_select"] if C > 64 else []) + ["la_state", "la_scan", "hybrid_main"]
    say(f"[path] W={W} C={C}: {names}")
    assert names == want


def test_fwd_is_deterministic(gpu_lib):
    cfg, seed = CASES["bf16_ragged_G4"]
    raw = workloads.make_prefill(cfg, seed)
    dev, _ = prepare(raw, torch.bfloat16)
    runs = [gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=64,
                        chunk=64, topk=16, return_scores=True, return_sel=True) for _ in range(2)]
    torch.cuda.synchronize()
    for key in ("out", "scores", "sel_idx"):
        assert torch.equal(runs[0][key], runs[1][key]), key


def test_empty_sequence_is_noop(gpu_lib):
    q = torch.zeros((1, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, 64, 128), dtype=torch.float32, device="cuda")
    res = gpu_lib.fwd(q, k, k, w, w, window=64, chunk=64, topk=16)
    assert res["out"].shape == (1, 0, 4, 128)


ROUTE_CASES = {
    "C64": (make_case("q", 1, 400, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 25),
    # the uniform criterion's offsets depend on C; selection over 128 keys
    "C128": (make_case("q", 1, 700, 8, 2, 128, 128, 128, 24, outlier_frac=0.02, heavy_scale=6.0), 39),
}
ROUTE_NAMES = ["diagonal", "qk", "keynorm", "uniform", "random"]


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("route", ROUTE_NAMES)
@pytest.mark.parametrize("shape", list(ROUTE_CASES))
def test_routing_criteria_match_oracle(gpu_lib, shape, route, general):
    """The routing criteria the pages compare with Self-Saliency: same scores,
    same selections (or near-ties the oracle adopts), same outputs."""
    cfg, seed = ROUTE_CASES[shape]
    say(f"[route] {route} {shape} general={general} shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch.bfloat16)
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                      topk=lam, return_scores=True, return_sel=True, general=general, route=route)
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam, route=route)
    sigma = O.window_scores(ref["q"], ref["k"], p, cfg["n_kv_heads"])
    gs = res["scores"].cpu().numpy()
    serr = float(np.max(np.abs(gs - sigma) / np.maximum(1.0, np.abs(sigma))))
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    osel, _ = O.select_chunks(sigma, p)
    n_bad, worst = check_selection(gsel, sigma, osel, C)
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p,
                     sel_override=gsel if n_bad else None, scores=sigma)
    out = res["out"].double().cpu().numpy()
    err = rel_l2(out, o["out"])
    say(f"  score max rel err {serr:.2e}; {n_bad} near-tie chunks; out rel-L2 {err:.3e}")
    assert serr <= 1e-4
    if route in ("uniform", "random"):
        np.testing.assert_array_equal(gsel, osel)
    assert err <= BF16_TOL
    check_rows(out, o["out"], row_tol("bf16"))


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
@pytest.mark.parametrize("route", ["saliency", "keynorm"])
@pytest.mark.parametrize("chunk,lam", [(64, 20), (128, 80)], ids=["C64", "C128"])
def test_selection_with_exact_ties(gpu_lib, chunk, lam, route, general):
    """Every token of a KV head carries the same key (and every query head the
    same query), so every full-window score in a chunk is the same number:
    the top-lambda threshold falls inside one run of equal keys and the lower
    positions must win, as the oracle's stable order says (with C = 128 and
    lambda = 80 the kept run spans both 64-key halves of a chunk)."""
    C = chunk
    cfg = make_case("t", 1, 300, 8, 2, 128, C, C, lam)
    raw = workloads.make_prefill(cfg, 32)
    raw["q"][:] = raw["q"][:, :1]
    raw["k"][:] = raw["k"][:, :1]
    dev, ref = prepare(raw, torch.bfloat16)
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=C, chunk=C,
                      topk=lam, return_scores=True, return_sel=True, general=general, route=route)
    torch.cuda.synchronize()
    p = O.Params(window=C, chunk=C, topk=lam, route=route)
    sigma = O.window_scores(ref["q"], ref["k"], p, 2)
    osel, _ = O.select_chunks(sigma, p)
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    if route == "keynorm":
        # one key norm per KV head: exact ties everywhere, the first lam positions win
        first = np.arange(lam)[None, None, None, :] + C * np.arange(300 // C)[None, None, :, None]
        np.testing.assert_array_equal(gsel, np.broadcast_to(first, gsel.shape))
        np.testing.assert_array_equal(gsel, osel)
    else:
        # the Self-Saliency of equal full-window rows agrees to the last bits
        # only: the near-tie protocol decides, and must find nothing else
        n_bad, worst = check_selection(gsel, sigma, osel, C)
        say(f"  {n_bad} chunks differ by near-ties (worst margin {worst:.2g})")
