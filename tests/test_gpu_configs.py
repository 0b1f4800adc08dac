"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the kernels the library picks for the shape):

* Llama-3-8B-shaped prefill layers (32 query / 8 KV heads, d = 128, W = C = 64):
  4K with topk 16, 16K with topk 32 plus a needle pair, 8 x 2K with topk 16.
  Every selected position and every group score is compared; outputs are
  compared on sampled query rows that the oracle evaluates one by one.
* The batched decode step (64 sequences at position 16384, 8160 selected
  rows per stream): outputs of sampled sequences over consecutive steps.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import BF16_TOL, ROW_TOL_BF16, check_rows, check_selection, prepare, rel_l2, sampled_rows, say

pytestmark = pytest.mark.gpu

PREFILL = ["prefill_4k", "prefill_16k", "train_8x2k"]


@pytest.mark.parametrize("name", PREFILL)
def test_prefill_config_matches_oracle(gpu_lib, name):
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    say(f"[config] {name} shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch.bfloat16)
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    B, N, Hkv = cfg["batch"], cfg["seqlen"], cfg["n_kv_heads"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W,
                      chunk=C, topk=lam, return_scores=True, return_sel=True)
    torch.cuda.synchronize()
    p = O.Params(window=W, chunk=C, topk=lam)
    sigma = O.window_scores(ref["q"], ref["k"], p, Hkv)
    osel, _ = O.select_chunks(sigma, p)
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    n_bad, worst = check_selection(gsel, sigma, osel, C)
    say(f"  selection: {gsel.size // lam} chunk decisions, {n_bad} near-tie swaps (worst {worst:.2g})")
    gs = res["scores"].cpu().numpy()
    serr = float(np.max(np.abs(gs - sigma) / np.maximum(1.0, np.abs(sigma))))
    if raw["needle"] is not None:
        kp = raw["needle"]["key_pos"][0]
        hit = [(kp in set(gsel[0, g, kp // C].tolist())) for g in range(Hkv)]
        say(f"  needle key at {kp}: selected in {sum(hit)}/{Hkv} KV heads (diagnostic)")
    rows = sampled_rows(B, N, C, n_per_batch=24, seed=seed,
                        extra=[N - 1] if raw["needle"] is not None else ())
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p, rows=rows,
                     sel_override=gsel if n_bad else None, scores=sigma)
    bi = np.array([r[0] for r in rows])
    ti = np.array([r[1] for r in rows])
    got = res["out"][bi, ti].double().cpu().numpy()
    want = o["out"][bi, ti]
    err = rel_l2(got, want)
    say(f"  {len(rows)} sampled rows: rel-L2 {err:.3e}; score max rel err {serr:.2e}")
    assert err <= BF16_TOL
    check_rows(got, want, ROW_TOL_BF16)
    assert serr <= 1e-4


def test_prefill_4k_two_chunk_window_matches_oracle(gpu_lib):
    """The 4K Llama-3-8B-shaped prefill with the pages' full-RULER window
    (W = 128 over chunks of 64, top-16) on the matrix-core path: every
    selection and group score compared, sampled rows evaluated by the oracle."""
    cfg = dict(workloads.CONFIGS["prefill_4k"], window=128)
    seed = workloads.seed_of("prefill_4k")
    say(f"[config] prefill_4k W=128 shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch.bfloat16)
    B, N, Hkv, C = cfg["batch"], cfg["seqlen"], cfg["n_kv_heads"], cfg["chunk"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=128,
                      chunk=C, topk=16, return_scores=True, return_sel=True)
    torch.cuda.synchronize()
    p = O.Params(window=128, chunk=C, topk=16)
    sigma = O.window_scores(ref["q"], ref["k"], p, Hkv)
    osel, _ = O.select_chunks(sigma, p)
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    n_bad, worst = check_selection(gsel, sigma, osel, C)
    serr = float(np.max(np.abs(res["scores"].cpu().numpy() - sigma) / np.maximum(1.0, np.abs(sigma))))
    rows = sampled_rows(B, N, C, n_per_batch=24, seed=seed, extra=[127, 128, 191, 192])
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p, rows=rows,
                     sel_override=gsel if n_bad else None, scores=sigma)
    bi = np.array([r[0] for r in rows])
    ti = np.array([r[1] for r in rows])
    got = res["out"][bi, ti].double().cpu().numpy()
    err = rel_l2(got, o["out"][bi, ti])
    say(f"  {n_bad} near-tie swaps; score max rel err {serr:.2e}; {len(rows)} sampled rows: rel-L2 {err:.3e}")
    assert err <= BF16_TOL
    check_rows(got, o["out"][bi, ti], ROW_TOL_BF16)
    assert serr <= 1e-4


def test_ragged_multi_sequence_prefill_matches_oracle(gpu_lib):
    """A 4K+37-token, two-sequence prefill on the matrix-core path: several
    runs of chunks in the linear-state kernel, a ragged last chunk, every
    selection compared and sampled rows evaluated by the oracle."""
    cfg = dict(batch=2, seqlen=4096 + 37, n_q_heads=8, n_kv_heads=4, head_dim=128, window=64,
               chunk=64, topk=16, dtype="bf16", outlier_frac=0.01, heavy_scale=6.0)
    seed = 41
    say(f"[config] ragged two-sequence 4K+37 shape={workloads.shape_of(cfg)} seed={seed}")
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch.bfloat16)
    B, N, Hkv, C = cfg["batch"], cfg["seqlen"], cfg["n_kv_heads"], cfg["chunk"]
    res = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=64,
                      chunk=C, topk=16, return_scores=True, return_sel=True)
    torch.cuda.synchronize()
    p = O.Params(window=64, chunk=C, topk=16)
    sigma = O.window_scores(ref["q"], ref["k"], p, Hkv)
    osel, _ = O.select_chunks(sigma, p)
    gsel = res["sel_idx"].cpu().numpy().astype(np.int64)
    n_bad, worst = check_selection(gsel, sigma, osel, C)
    rows = sampled_rows(B, N, C, n_per_batch=20, seed=seed, extra=[N - 1, N - 37, 4095])
    o = O.fwd_direct(ref["q"], ref["k"], ref["v"], ref["wphi_q"], ref["wphi_k"], p, rows=rows,
                     sel_override=gsel if n_bad else None, scores=sigma)
    bi = np.array([r[0] for r in rows])
    ti = np.array([r[1] for r in rows])
    got = res["out"][bi, ti].double().cpu().numpy()
    err = rel_l2(got, o["out"][bi, ti])
    say(f"  {n_bad} near-tie swaps; {len(rows)} sampled rows: rel-L2 {err:.3e}")
    assert err <= BF16_TOL
    check_rows(got, o["out"][bi, ti], ROW_TOL_BF16)


def test_decode_config_matches_oracle(gpu_lib):
    name = "decode_b64_16k"
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    n_steps = 3
    say(f"[config] {name} steps={n_steps} seed={seed}")
    B, Hq, Hkv, d = cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    W, C, lam, cap = cfg["window"], cfg["chunk"], cfg["topk"], cfg["sel_cap"]
    full = workloads.make_decode_cache(cfg, seed)
    gc = gpu_lib.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C, topk=lam,
                             sel_cap=cap, pos=cfg["pos"])
    for key, arr in full.items():
        t = getattr(gc, key)
        t.copy_(torch.from_numpy(arr).to(t.dtype))
    del full
    toks = workloads.make_decode_tokens(cfg, seed, n_steps)
    bs = [0, 37, 63]
    part = workloads.make_decode_cache(cfg, seed, batches=bs)
    oc = {}
    for key, arr in part.items():
        if key in ("win_k", "win_v", "sel_k", "sel_v"):
            oc[key] = torch.from_numpy(arr).to(torch.bfloat16).double().numpy()
        elif key in ("win_route", "sel_count"):
            oc[key] = arr.astype(np.int64) if key == "sel_count" else arr.copy()
        else:
            oc[key] = arr.astype(np.float64)
    oc["pos"] = cfg["pos"]
    wq = torch.from_numpy(toks["wphi_q"]).cuda()
    wk = torch.from_numpy(toks["wphi_k"]).cuda()
    p = O.Params(window=W, chunk=C, topk=lam)
    for s in range(n_steps):
        qt = torch.from_numpy(toks["q"][s]).to(torch.bfloat16)
        kt = torch.from_numpy(toks["k"][s]).to(torch.bfloat16)
        vt = torch.from_numpy(toks["v"][s]).to(torch.bfloat16)
        out = gpu_lib.decode_step(qt[:, None].cuda(), kt[:, None].cuda(), vt[:, None].cuda(), wq,
                                  wk, gc)
        want = O.decode_step(oc, qt[bs].double().numpy(), kt[bs].double().numpy(),
                             vt[bs].double().numpy(), toks["wphi_q"].astype(np.float64),
                             toks["wphi_k"].astype(np.float64), p)
        torch.cuda.synchronize()
        got = out[bs, 0].double().cpu().numpy()
        err = rel_l2(got, want)
        say(f"  step {s} (t={cfg['pos'] + s}): sampled sequences {bs} rel-L2 {err:.3e}")
        assert err <= BF16_TOL
        check_rows(got, want, ROW_TOL_BF16, what=f"step {s}")
    np.testing.assert_array_equal(gc.sel_count.cpu().numpy()[bs], oc["sel_count"])
