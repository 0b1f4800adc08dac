"""Benchmark of the STILL hybrid-attention layer on one MI355X.

One step = one whole forward of the operator (window scores, per-chunk
selection, sparse softmax + NP-Map linear attention, aggregation) over the
Llama-3-8B-shaped 16K-token prefill (batch 1, 32 query / 8 KV heads,
head_dim 128, window = chunk = 64, top-32 per chunk, bf16 storage with fp32
accumulation), inputs resident in HBM.  The decode step (batch 64 at
position 16384) is timed the same way and reported in the "decode" object,
and its serving form (the same batch with one position per sequence) in
"decode_ragged"; the backward pass (gradients w.r.t. q, k, v and the NP-Map
projections) on the 8 x 2048 training batch in "backward"; the future-KV-utility
diagnostic of the routing criteria on the 4K prefill in "future_kv_utility".

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on
the launch stream by the library's *_timed entry points; the roofline uses
the dominant kernel's algorithmic work per launch over its average duration.
The CPU baseline is the float64 oracle on a bounded sample of the same
workload, timed on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "hybrid-attn layer tokens/s (Llama-3-8B shape, 16K prefill; decode) + % roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources that define each measured kernel: a stored counter reading is used
# only while their hash is unchanged
KERNEL_SOURCES = {
    "hybrid_main": ["hybrid_sparse_softmax_amd/csrc/prefill_mfma.hip",
                    "hybrid_sparse_softmax_amd/csrc/mfma_common.h",
                    "hybrid_sparse_softmax_amd/csrc/mfma_tiles.h",
                    "hybrid_sparse_softmax_amd/csrc/device_common.h"],
    "dec_stream": ["hybrid_sparse_softmax_amd/csrc/decode_fast.hip",
                   "hybrid_sparse_softmax_amd/csrc/device_common.h"],
    "bwd_query": ["hybrid_sparse_softmax_amd/csrc/backward.hip",
                  "hybrid_sparse_softmax_amd/csrc/device_common.h",
                  "hybrid_sparse_softmax_amd/csrc/row_ops.h"],
    "bwd_dq": ["hybrid_sparse_softmax_amd/csrc/backward_mfma.hip",
               "hybrid_sparse_softmax_amd/csrc/mfma_tiles.h",
               "hybrid_sparse_softmax_amd/csrc/mfma_common.h",
               "hybrid_sparse_softmax_amd/csrc/device_common.h"],
    "bwd_kv_sel": ["hybrid_sparse_softmax_amd/csrc/backward_mfma.hip",
                   "hybrid_sparse_softmax_amd/csrc/mfma_tiles.h",
                   "hybrid_sparse_softmax_amd/csrc/mfma_common.h",
                   "hybrid_sparse_softmax_amd/csrc/device_common.h"],
}


def sources_sha(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each divided by what the same counter
    reads per byte of a plain copy), or None when there is no reading for
    this workload or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("workload") != workload or rec.get("sources_sha256") != sources_sha(kernel):
        return None
    fetch = rec["fetch_kib"] * 1024.0 / rec["copy_fetch_per_byte"]
    write = rec["write_kib"] * 1024.0 / rec["copy_write_per_byte"]
    return round(fetch + write)
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (counted once per mathematical operation; exp/log excluded)
# ---------------------------------------------------------------------------
def prefill_flops(cfg: dict, sel_idx: np.ndarray) -> dict:
    B, N, Hq, Hkv = cfg["batch"], cfg["seqlen"], cfg["n_q_heads"], cfg["n_kv_heads"]
    d = cfg["head_dim"]
    fd = d
    W, C = cfg["window"], cfg["chunk"]
    G = Hq // Hkv
    t = np.arange(N)
    win_pairs = float(np.minimum(t + 1, W).sum()) * Hq * B
    r_end = np.maximum(0, t - W + 1)
    sel_pairs = 0.0
    for b in range(B):
        for g in range(Hkv):
            pos = np.sort(sel_idx[b, g].reshape(-1))
            sel_pairs += float(np.searchsorted(pos, r_end, side="left").sum()) * G
    per_qh_la = 2 * fd * d + 2 * C * fd + 2 * C * d + 2 * fd
    return dict(
        win=4.0 * d * win_pairs,                     # QK^T + PV over window pairs
        sel=4.0 * d * sel_pairs,                     # QK^T + PV over visible selected pairs
        la_read=float(per_qh_la) * N * Hq * B,       # phi_q.P + intra-chunk LA block
        np_q=float(fd * d) * N * Hq * B,             # NP-Map projection of queries
        np_k=float(fd * d) * N * Hkv * B,            # NP-Map projection of keys
        la_state=float(2 * fd * d + 2 * fd) * N * Hkv * B,   # per-chunk phi_k^T V, z
        score_qk=2.0 * d * win_pairs,                # window logits for the scores
    )


KERNEL_FLOPS = {
    # kernel launch name -> which algorithmic terms that kernel computes
    "main_general": ("win", "sel", "la_read"),
    "hybrid_main": ("win", "sel", "la_read", "np_q"),
}


def decode_bytes(cfg: dict, sel_count: np.ndarray) -> dict:
    """HBM bytes of one decode step that the method must move."""
    d, W, Hq, Hkv, B = cfg["head_dim"], cfg["window"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["batch"]
    e = 2  # bf16
    sel = float(sel_count.sum()) * 2 * d * e             # selected K and V rows
    ring = float(B * Hkv) * W * 2 * d * e
    state = float(B * Hkv) * (d * d + d) * 4 * 2          # S, z read + (LA eviction) write
    qo = float(B * Hq) * d * e * 2 + float(B * Hkv) * 2 * d * e
    return dict(sel=sel, ring=ring, state=state, qo=qo, total=sel + ring + state + qo)


# ---------------------------------------------------------------------------
def bench_prefill(still, torch, name, steps, warmup):
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    t0 = time.time()
    raw = workloads.make_prefill(cfg, seed)
    dev = {k: torch.from_numpy(raw[k]).to(torch.bfloat16).cuda() for k in ("q", "k", "v")}
    for k in ("wphi_q", "wphi_k"):
        dev[k] = torch.from_numpy(raw[k]).cuda()
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s")
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    kw = dict(window=W, chunk=C, topk=lam)
    out = torch.empty_like(dev["q"])
    sh = still.make_shape(batch=cfg["batch"], seqlen=cfg["seqlen"], n_q_heads=cfg["n_q_heads"],
                          n_kv_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], **kw)
    ws = torch.empty(still.fwd_workspace_size(sh), dtype=torch.uint8, device="cuda")
    args = (dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"])
    first = still.fwd(*args, **kw, return_sel=True, workspace=ws)
    sel_idx = first["sel_idx"].cpu().numpy()
    for _ in range(warmup):
        still.fwd(*args, **kw, out=out, workspace=ws)
    timers = [still.LaunchTimer() for _ in range(steps)]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        still.fwd(*args, **kw, out=out, workspace=ws, timer=timers[i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per = {}
    for tm in timers:
        for kname, dur in tm.durations_ms():
            per.setdefault(kname, []).append(dur)
    kern = {k: float(np.mean(v)) for k, v in per.items()}
    log(f"[bench] {name}: {ms:.3f} ms/step; kernels (ms): " +
        ", ".join(f"{k}={v:.3f}" for k, v in kern.items()))
    flops = prefill_flops(cfg, sel_idx)
    dom = max(kern, key=kern.get)
    terms = KERNEL_FLOPS.get(dom)
    roof = None
    if terms:
        alg = sum(flops[t] for t in terms)
        achieved = alg / (kern[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, name), "kernel": dom, "avg_ms": round(kern[dom], 4),
                "algorithmic_flop_per_launch": alg}
    total_alg = sum(v for k, v in flops.items() if k != "score_qk")
    return dict(cfg=cfg, raw=raw, ms=ms, kern=kern, roof=roof, flops=flops,
                total_alg=total_alg, tokens=cfg["batch"] * cfg["seqlen"])


def bench_decode(still, torch, steps, warmup):
    name = "decode_b64_16k"
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    B, Hq, Hkv, d = cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    t0 = time.time()
    full = workloads.make_decode_cache(cfg, seed)
    cache = still.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=cfg["window"],
                              chunk=cfg["chunk"], topk=cfg["topk"], sel_cap=cfg["sel_cap"],
                              pos=cfg["pos"])
    for key, arr in full.items():
        t = getattr(cache, key)
        t.copy_(torch.from_numpy(arr).to(t.dtype))
    del full
    n_tok = warmup + steps
    toks = workloads.make_decode_tokens(cfg, seed, n_tok)
    q = torch.from_numpy(toks["q"]).to(torch.bfloat16).cuda()
    k = torch.from_numpy(toks["k"]).to(torch.bfloat16).cuda()
    v = torch.from_numpy(toks["v"]).to(torch.bfloat16).cuda()
    wq = torch.from_numpy(toks["wphi_q"]).cuda()
    wk = torch.from_numpy(toks["wphi_k"]).cuda()
    log(f"[bench] {name}: cache ready in {time.time() - t0:.1f}s")
    sh = still.make_shape(batch=B, seqlen=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                          window=cfg["window"], chunk=cfg["chunk"], topk=cfg["topk"])
    ws = torch.empty(still.decode_workspace_size(sh, cfg["sel_cap"]), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    qs = [q[i][:, None].contiguous() for i in range(n_tok)]
    ks = [k[i][:, None].contiguous() for i in range(n_tok)]
    vs = [v[i][:, None].contiguous() for i in range(n_tok)]
    for i in range(warmup):
        still.decode_step(qs[i], ks[i], vs[i], wq, wk, cache, out=out, workspace=ws)
    sel_before = cache.sel_count.cpu().numpy().copy()
    timers = [still.LaunchTimer() for _ in range(steps)]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        j = warmup + i
        still.decode_step(qs[j], ks[j], vs[j], wq, wk, cache, out=out, workspace=ws, timer=timers[i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    sel_after = cache.sel_count.cpu().numpy()
    per = {}
    for tm in timers:
        for kname, dur in tm.durations_ms():
            per.setdefault(kname, []).append(dur)
    kern = {k: float(np.mean(v)) for k, v in per.items()}
    log(f"[bench] {name}: {ms:.3f} ms/step; kernels (ms): " +
        ", ".join(f"{k}={v:.3f}" for k, v in kern.items()))
    mid = (sel_before.astype(np.float64) + sel_after) / 2
    by = decode_bytes(cfg, mid)
    dom = max(kern, key=kern.get)
    # the general path's split-KV kernel moves only the selected rows; the
    # fast path's stream kernel does every step's memory work but the merge
    dom_bytes = by["sel"] + float(B * Hq) * d * 2 if dom.startswith("decode_sel") else by["total"]
    achieved = dom_bytes / (kern[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom, name), "kernel": dom,
            "avg_ms": round(kern[dom], 4), "algorithmic_bytes_per_launch": dom_bytes}
    step_gbs = by["total"] / (ms * 1e-3) / 1e9
    t_first = cfg["pos"] + warmup
    chunk_ends = sum(1 for t in range(t_first, t_first + steps) if t % cfg["chunk"] == cfg["chunk"] - 1)
    return {"metric": "decode tokens/s (batch 64 at position 16384)", "value": round(B / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
            "timed_positions": [t_first, t_first + steps - 1], "chunk_end_steps_timed": chunk_ends,
            "config": {"workload": "decode_b64_16k: batch 64, one token per sequence at position "
                       "16384, 32 q / 8 KV heads, d 128, window 64, chunk 64, top-32, "
                       "8160 selected rows per (sequence, KV head), fp32 128x128 state",
                       "batch": B, "pos": cfg["pos"]},
            "step_algorithmic_bytes": by["total"], "step_GBps": round(step_gbs, 1),
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()}, "roofline": roof}


def bench_decode_ragged(still, torch, steps, warmup):
    """The decode step in its serving form: the same batch-64 shape with one
    position per sequence (multiples of 64 drawn from [1024, 16384]), each
    sequence's selected list as long as its position implies."""
    name = "decode_b64_16k"
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    B, Hq, Hkv, d = cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    positions = workloads.decode_positions(cfg, seed)
    t0 = time.time()
    full = workloads.make_decode_cache(cfg, seed, positions=positions)
    cache = still.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=cfg["window"],
                              chunk=cfg["chunk"], topk=cfg["topk"], sel_cap=cfg["sel_cap"])
    for key, arr in full.items():
        t = getattr(cache, key)
        t.copy_(torch.from_numpy(arr).to(t.dtype))
    del full
    n_tok = warmup + steps
    toks = workloads.make_decode_tokens(cfg, seed, n_tok)
    q = torch.from_numpy(toks["q"]).to(torch.bfloat16).cuda()
    k = torch.from_numpy(toks["k"]).to(torch.bfloat16).cuda()
    v = torch.from_numpy(toks["v"]).to(torch.bfloat16).cuda()
    wq = torch.from_numpy(toks["wphi_q"]).cuda()
    wk = torch.from_numpy(toks["wphi_k"]).cuda()
    log(f"[bench] {name} ragged: cache ready in {time.time() - t0:.1f}s "
        f"(positions {int(positions.min())}..{int(positions.max())}, mean {positions.mean():.0f})")
    pos = torch.from_numpy(positions).cuda()
    top = int(positions.max())
    sh = still.make_shape(batch=B, seqlen=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                          window=cfg["window"], chunk=cfg["chunk"], topk=cfg["topk"])
    ws = torch.empty(still.decode_workspace_size(sh, cfg["sel_cap"]), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    qs = [q[i][:, None].contiguous() for i in range(n_tok)]
    ks = [k[i][:, None].contiguous() for i in range(n_tok)]
    vs = [v[i][:, None].contiguous() for i in range(n_tok)]
    for i in range(warmup):
        still.decode_step_ragged(qs[i], ks[i], vs[i], wq, wk, cache, pos, top + i, out=out, workspace=ws)
    sel_before = cache.sel_count.cpu().numpy().copy()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        j = warmup + i
        still.decode_step_ragged(qs[j], ks[j], vs[j], wq, wk, cache, pos, top + j, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    mid = (sel_before.astype(np.float64) + cache.sel_count.cpu().numpy()) / 2
    by = decode_bytes(cfg, mid)
    gbs = by["total"] / (ms * 1e-3) / 1e9
    log(f"[bench] {name} ragged: {ms:.3f} ms/step, {gbs:.0f} GB/s algorithmic")
    C = cfg["chunk"]
    chunk_ends = int(sum(((positions + warmup + i) % C == C - 1).sum() for i in range(steps)))
    return {"metric": "decode tokens/s, ragged positions (batch 64)", "value": round(B / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
            "chunk_end_sequence_steps_timed": chunk_ends,
            "config": {"workload": "decode_b64 ragged: batch 64, one token per sequence, positions "
                       "multiples of 64 drawn from [1024, 16384], 32 q / 8 KV heads, d 128, window 64, "
                       "chunk 64, top-32", "batch": B,
                       "positions": {"min": int(positions.min()), "max": int(positions.max()),
                                     "mean": round(float(positions.mean()), 1)}},
            "step_algorithmic_bytes": by["total"], "step_GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs at 2.4 GHz)


def backward_flops(cfg: dict, sel_idx: np.ndarray) -> dict:
    """Algorithmic flops of the backward (exp excluded), per kernel that does
    them, and "method": the whole step counted once per mathematical
    operation.  A softmax pair (query, visible key) costs the method 10d: the
    logit, dout . v, and the three products dS k, dS q, P dout.  The
    matrix-core kernels recompute the logit and dout . v on each side: the
    dq kernel does 6d per pair, the key kernels 8d (window pairs in
    bwd_kv_win, pairs of a selected key and a query after its window in
    bwd_kv_sel); their first pass is the forward's main kernel (4d per pair,
    the linear read-out, the NP-Map of the queries) plus dout . out.  Linear
    terms: S_t dout per query head (2 d' d), the chunk sums c phi_q dout^T per
    query head (2 d' d), U^T phi_k and U v per routed linear key (4 d' d),
    explicit pairs of the partly covered chunk (query side 2d + 2d' per pair
    on the matrix cores, whose first pass has the normaliser; 4d + 4d' in the
    fp32 kernel; key side 4d + 4d'); NP-Map backward 2 d' d and its
    projection gradient d' d per token-head.  On the matrix cores the dq
    kernel also runs the queries' NP-Map backward and the key linear kernel
    the keys' (no np_vjp launches); their recomputation of u = P x is not
    counted, nor, when the dq kernel starts from the forward's statistics
    (no first pass), its NP-Map of the queries."""
    B, N, Hq, Hkv = cfg["batch"], cfg["seqlen"], cfg["n_q_heads"], cfg["n_kv_heads"]
    d = fd = cfg["head_dim"]
    W, C = cfg["window"], cfg["chunk"]
    lam = min(cfg["topk"], C)
    G = Hq // Hkv
    t = np.arange(N)
    win_pairs = float(np.minimum(t + 1, W).sum()) * Hq * B
    r_end = np.maximum(0, t - W + 1)
    c_full = r_end // C
    n_full = N // C
    sel_pairs = q_part = k_part = la_keys = 0.0
    for b in range(B):
        for g in range(Hkv):
            pos = np.sort(sel_idx[b, g].reshape(-1)) if lam > 0 else np.zeros(0, np.int64)
            sel_pairs += float(np.searchsorted(pos, r_end, side="left").sum()) * G
            la = np.ones(N, np.int64)
            if lam > 0:
                la[n_full * C:] = 0
                la[pos] = 0
            cum = np.concatenate([[0], np.cumsum(la)])
            q_part += float((cum[r_end] - cum[c_full * C]).sum()) * G
            j = np.arange(max(0, N - W))
            jl = j[la[j] == 1]
            t1 = np.minimum(N - 1, ((jl + W) // C + 1) * C - 1)
            k_part += float((t1 - (jl + W) + 1).sum()) * G
            la_keys += float(jl.size)
    sa = win_pairs + sel_pairs
    tok_q, tok_k = float(B * N * Hq), float(B * N * Hkv)
    lin_q = 2.0 * fd * d * tok_q + (4.0 * d + 4.0 * fd) * q_part
    lin_k = 4.0 * fd * d * la_keys + (4.0 * d + 4.0 * fd) * k_part
    fwd_like = 4.0 * d * sa + (2 * fd * d + 2 * C * fd + 2 * C * d + 2 * fd) * tok_q + fd * d * tok_q
    out = dict(
        # matrix-core path
        bwd_stats=fwd_like + 2.0 * d * tok_q,
        bwd_dq=6.0 * d * sa + 2.0 * fd * d * tok_q + (2.0 * d + 2.0 * fd) * q_part + 2.0 * fd * d * tok_q,
        bwd_kv_win=8.0 * d * win_pairs,
        bwd_kv_sel=8.0 * d * sel_pairs,
        bwd_key_la=lin_k + 2.0 * fd * d * tok_k,
        # general path
        bwd_query=6.0 * d * sa + lin_q,
        bwd_key_win=8.0 * d * win_pairs + lin_k,
        bwd_key_sel=8.0 * d * sel_pairs,
        # both
        bwd_uchunk=2.0 * fd * d * tok_q + 2.0 * fd * tok_q,
        np_vjp_q=2.0 * fd * d * tok_q,
        np_vjp_k=2.0 * fd * d * tok_k,
        dw_q=1.0 * fd * d * tok_q,
        dw_k=1.0 * fd * d * tok_k,
    )
    out["method"] = (10.0 * d * sa + lin_q + lin_k + out["bwd_uchunk"]
                     + out["np_vjp_q"] + out["np_vjp_k"] + out["dw_q"] + out["dw_k"]
                     + (2 * fd * d + 2 * fd) * tok_k)
    return out


MFMA_KERNELS = {"bwd_stats", "bwd_dq", "bwd_kv_win", "bwd_kv_sel", "bwd_uchunk", "bwd_key_la",
                "dw_q", "dw_k"}


def bench_backward(still, torch, steps, warmup, name="train_8x2k"):
    """The backward pass on the training-shaped batch (8 sequences of 2048
    tokens): gradients w.r.t. q, k, v and both NP-Map projections under the
    forward's own routing, dout ~ N(0, 1), started from the forward's output
    and statistics (the time from the routing alone, with the first pass
    that recomputes them, is reported beside it)."""
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    raw = workloads.make_prefill(cfg, seed)
    dev = {k: torch.from_numpy(raw[k]).to(torch.bfloat16).cuda() for k in ("q", "k", "v")}
    for k in ("wphi_q", "wphi_k"):
        dev[k] = torch.from_numpy(raw[k]).cuda()
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(torch.bfloat16).cuda()
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    kw = dict(window=W, chunk=C, topk=lam)
    args = (dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"])
    # the training pairing: the forward hands the backward its routing, its
    # output, its per-query statistics and its workspace (the keys' NP-Map
    # features and the linear prefixes)
    fw = still.fwd(*args, **kw, return_sel=True, return_stats=True, return_workspace=True)
    sel = fw["sel_idx"]
    saved = dict(out=fw["out"], stats=fw["stats"], fwd_workspace=fw["workspace"])
    sh = still.make_shape(batch=cfg["batch"], seqlen=cfg["seqlen"], n_q_heads=cfg["n_q_heads"],
                          n_kv_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], **kw)
    ws = torch.empty(still.bwd_workspace_size(sh), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def time_bwd(extra, timers=None):
        for _ in range(warmup):
            still.bwd(*args, sel, dout, **kw, workspace=ws, **extra)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            still.bwd(*args, sel, dout, **kw, workspace=ws, **extra,
                      timer=timers[i] if timers else None)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # from the routing alone (a first pass recomputes the statistics)
    recompute_ms = time_bwd({})
    log(f"[bench] {name} backward from the routing alone: {recompute_ms:.3f} ms/step")
    timers = [still.LaunchTimer() for _ in range(steps)]
    ms = time_bwd(saved, timers)
    per = {}
    for tm in timers:
        for kname, dur in tm.durations_ms():
            per.setdefault(kname, []).append(dur)
    kern = {k: float(np.mean(v)) for k, v in per.items()}
    log(f"[bench] {name} backward: {ms:.3f} ms/step; kernels (ms): " +
        ", ".join(f"{k}={v:.3f}" for k, v in kern.items()))
    # the forward of the same batch (writing the statistics), for the
    # backward / forward ratio
    fws = torch.empty(still.fwd_workspace_size(sh), dtype=torch.uint8, device="cuda")
    fout = torch.empty_like(dev["q"])
    fst = torch.empty_like(fw["stats"])
    for _ in range(warmup):
        still.fwd(*args, **kw, out=fout, workspace=fws, stats=fst)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        still.fwd(*args, **kw, out=fout, workspace=fws, stats=fst)
    e1.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / steps
    log(f"[bench] {name} forward: {fwd_ms:.3f} ms/step; backward / forward {ms / fwd_ms:.2f}")
    fl = backward_flops(cfg, sel.cpu().numpy())
    dom = max(kern, key=kern.get)
    roof = None
    if dom in fl:
        mfma = dom in MFMA_KERNELS
        peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_VALU_TFLOPS
        achieved = fl[dom] / (kern[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma" if mfma else "alu", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom, name), "kernel": dom, "avg_ms": round(kern[dom], 4),
                "algorithmic_flop_per_launch": fl[dom]}
    mfma_kernels = {k: {"ms": round(kern[k], 4), "TFLOPs": round(fl[k] / (kern[k] * 1e-3) / 1e12, 1),
                        "frac_of_bf16_peak": round(fl[k] / (kern[k] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
                    for k in MFMA_KERNELS if k in kern}
    total = fl["method"]
    tokens = cfg["batch"] * cfg["seqlen"]
    return {"metric": "backward tokens/s (8 x 2048 training batch)",
            "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
            "config": {"workload": f"{name}: batch {cfg['batch']}, seq {cfg['seqlen']}, "
                       f"{cfg['n_q_heads']} q / {cfg['n_kv_heads']} KV heads, d {cfg['head_dim']}, "
                       f"window {W}, chunk {C}, top-{lam}; gradients of q, k, v, both NP-Map "
                       "projections (fp32) under the forward's routing", "batch": cfg["batch"],
                       "seq_len": cfg["seqlen"]},
            "forward_ms": round(fwd_ms, 4), "backward_over_forward": round(ms / fwd_ms, 2),
            "from_forward_statistics": True, "from_forward_workspace": True, "recompute_statistics_ms": round(recompute_ms, 4),
            "whole_step_TFLOPs": round(total / (ms * 1e-3) / 1e12, 2),
            "whole_step_count": "method flops: 10d per softmax pair plus the linear and NP-Map terms",
            "matrix_core_kernels": mfma_kernels,
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()}, "roofline": roof}


def bench_n_scaling(still, torch, steps=5, warmup=2):
    """Prefill time against sequence length at a fixed selected-token budget
    (full text Sec. 3.3, complexity; App. A.4): m - W = 8192 selected rows per
    KV head, the per-chunk quota re-derived from each length,
    lambda(N) = floor((m - W) / ceil(N / C)) (capped at C), the 16K prefill's
    shape otherwise (32 / 8 heads, d 128, W = C = 64).  Once the budget is
    full (N >= 16K) every query sees at most W + m keys, so the time per
    token should stay flat and the step time grow linearly in N."""
    cfg = dict(workloads.CONFIGS["prefill_16k"])
    W, C = cfg["window"], cfg["chunk"]
    m = 8192 + W
    rows = []
    for N in (4096, 8192, 16384, 32768, 65536):
        lam = min(C, still.topk_for_budget(m, W, C, N))
        c = dict(cfg, seqlen=N, topk=lam)
        raw = workloads.make_prefill(c, workloads.seed_of("prefill_16k"))
        dev = {k: torch.from_numpy(raw[k]).to(torch.bfloat16).cuda() for k in ("q", "k", "v")}
        for k in ("wphi_q", "wphi_k"):
            dev[k] = torch.from_numpy(raw[k]).cuda()
        del raw
        kw = dict(window=W, chunk=C, topk=lam)
        sh = still.make_shape(batch=1, seqlen=N, n_q_heads=c["n_q_heads"], n_kv_heads=c["n_kv_heads"],
                              head_dim=c["head_dim"], **kw)
        ws = torch.empty(still.fwd_workspace_size(sh), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(dev["q"])
        args = (dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"])
        for _ in range(warmup):
            still.fwd(*args, **kw, out=out, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            still.fwd(*args, **kw, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        rows.append({"seq_len": N, "topk": lam, "ms": round(ms, 4), "ns_per_token": round(ms * 1e6 / N, 2)})
        log(f"[bench] n-scaling N={N} topk={lam}: {ms:.3f} ms ({ms * 1e6 / N:.1f} ns/token)")
        del dev, ws, out
    return {"budget_m": m, "window": W, "chunk": C, "rows": rows}


def bench_chunk_sweep(still, torch, steps=5, warmup=2, name="train_8x2k"):
    """Cost of one training step (forward + backward) against the chunk size
    (full text App. A.7.5, Table 14: C varied with the window spanning one
    chunk, W = C, and 16 selected tokens per chunk), on the 8 x 2048 training
    batch for the chunk sizes the matrix-core path takes (64, 128, 256); the
    backward starts from the forward's output, statistics and workspace."""
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    raw = workloads.make_prefill(cfg, seed)
    dev = {k: torch.from_numpy(raw[k]).to(torch.bfloat16).cuda() for k in ("q", "k", "v")}
    for k in ("wphi_q", "wphi_k"):
        dev[k] = torch.from_numpy(raw[k]).cuda()
    dout = torch.from_numpy(workloads.make_grad_out(cfg, seed)).to(torch.bfloat16).cuda()
    args = (dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"])
    lam = cfg["topk"]
    rows = []
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for C in (64, 128, 256):
        kw = dict(window=C, chunk=C, topk=lam)
        sh = still.make_shape(batch=cfg["batch"], seqlen=cfg["seqlen"], n_q_heads=cfg["n_q_heads"],
                              n_kv_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], **kw)
        fws = torch.empty(still.fwd_workspace_size(sh), dtype=torch.uint8, device="cuda")
        bws = torch.empty(still.bwd_workspace_size(sh), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(dev["q"])
        B, N = cfg["batch"], cfg["seqlen"]

        def step():
            fw = still.fwd(*args, **kw, out=out, workspace=fws, return_sel=True, return_stats=True)
            e_mid = torch.cuda.Event(enable_timing=True)
            e_mid.record()
            still.bwd(*args, fw["sel_idx"], dout, **kw, workspace=bws, out=out, stats=fw["stats"],
                      fwd_workspace=fws)
            return e_mid

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        fwd_ms = bwd_ms = 0.0
        for _ in range(steps):
            e0.record()
            mid = step()
            e1.record()
            torch.cuda.synchronize()
            fwd_ms += e0.elapsed_time(mid)
            bwd_ms += mid.elapsed_time(e1)
        fwd_ms /= steps
        bwd_ms /= steps
        ms = fwd_ms + bwd_ms
        rows.append({"chunk": C, "window": C, "topk": lam, "forward_ms": round(fwd_ms, 4),
                     "backward_ms": round(bwd_ms, 4), "step_ms": round(ms, 4),
                     "tokens_per_s": round(B * N / (ms * 1e-3), 1)})
        log(f"[bench] chunk sweep C=W={C} top-{lam}: forward {fwd_ms:.3f} + backward {bwd_ms:.3f} "
            f"= {ms:.3f} ms/step")
        del fws, bws, out
    return {"workload": f"{name} forward + backward, W = C, top-{lam} per chunk", "rows": rows}


def bench_utility(still, torch, name="prefill_4k"):
    """Future-KV-utility diagnostic (full text App. A.7.4, Table 12) on the
    4K prefill: the library's utilities of every remote key, then for each
    routing criterion the share of its selected remote tokens that are
    among as many keys ranked by utility (higher first, then lower
    position).  Synthetic inputs: the shares say how each criterion behaves
    on this distribution, not on a trained model."""
    cfg = workloads.CONFIGS[name]
    seed = workloads.seed_of(name)
    raw = workloads.make_prefill(cfg, seed)
    dev = {k: torch.from_numpy(raw[k]).to(torch.bfloat16).cuda() for k in ("q", "k", "v")}
    for k in ("wphi_q", "wphi_k"):
        dev[k] = torch.from_numpy(raw[k]).cuda()
    W, C, lam, N = cfg["window"], cfg["chunk"], cfg["topk"], cfg["seqlen"]
    still.future_kv_utility(dev["q"], dev["k"], window=W, chunk=C)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    u = still.future_kv_utility(dev["q"], dev["k"], window=W, chunk=C)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    u = u.cpu().numpy()
    elig = np.arange(max(0, N - W))
    shares = {}
    for route in still.ROUTES:
        sel = still.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                        topk=lam, return_sel=True, route=route)["sel_idx"].cpu().numpy()
        hit = tot = 0
        for b in range(sel.shape[0]):
            for g in range(sel.shape[1]):
                chosen = set(int(j) for j in sel[b, g].ravel() if j < elig.size)
                order = np.lexsort((elig, -u[b, g, elig]))
                top = set(elig[order[:len(chosen)]].tolist())
                hit += len(chosen & top)
                tot += len(chosen)
        shares[route] = round(hit / max(tot, 1), 4)
    log(f"[bench] {name} future-KV utility: {ms:.2f} ms; overlap " +
        ", ".join(f"{k}={v:.1%}" for k, v in shares.items()))
    return {"metric": "share of selected remote tokens among the top keys by future full-attention weight",
            "workload": f"{name}: batch {cfg['batch']}, seq {N}, {cfg['n_q_heads']} q / {cfg['n_kv_heads']} KV "
                        f"heads, window {W}, chunk {C}, top-{lam}; synthetic inputs",
            "utility_ms": round(ms, 3), "overlap": shares}


def cpu_baseline(raw, cfg, n_rows=12):
    """The oracle as it stands, on a bounded sample: group scores and
    selection over the whole sequence, then n_rows output rows evaluated one
    by one; tokens/s extrapolates the per-row cost to every row."""
    import oracle as O
    import torch
    from threadpoolctl import threadpool_info

    ref = {}
    for key in ("q", "k", "v"):
        ref[key] = torch.from_numpy(raw[key]).to(torch.bfloat16).double().numpy()
    wq, wk = raw["wphi_q"].astype(np.float64), raw["wphi_k"].astype(np.float64)
    p = O.Params(window=cfg["window"], chunk=cfg["chunk"], topk=cfg["topk"])
    B, N = cfg["batch"], cfg["seqlen"]
    t0 = time.perf_counter()
    sigma = O.window_scores(ref["q"], ref["k"], p, cfg["n_kv_heads"])
    O.select_chunks(sigma, p)
    t1 = time.perf_counter()
    rows = [(0, int(t)) for t in np.linspace(0, N - 1, n_rows).round()]
    O.fwd_direct(ref["q"], ref["k"], ref["v"], wq, wk, p, rows=rows, scores=sigma)
    t2 = time.perf_counter()
    per_row = (t2 - t1) / len(rows)
    est = (t1 - t0) + per_row * B * N
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(B * N / est, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"float64 numpy oracle: scores+selection over all {B * N} tokens "
                       f"({t1 - t0:.1f}s) plus {len(rows)} output rows evaluated one by one "
                       f"({t2 - t1:.1f}s), per-row cost extrapolated to all {B * N} rows; "
                       f"BLAS threads {threads}, elementwise numpy single-threaded")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_16k", choices=["prefill_4k", "prefill_16k", "train_8x2k"])
    ap.add_argument("--decode-steps", type=int, default=80,
                    help="timed decode steps (80 from position 16384 + warm-up cross the chunk "
                         "end at 16447, so a chunk-end top-k is inside the figure)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-utility", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-scaling", action="store_true",
                    help="skip the prefill-time-against-length sweep at a fixed budget")
    ap.add_argument("--no-chunk-sweep", action="store_true",
                    help="skip the training-step cost against the chunk size")
    ap.add_argument("--chunk-sweep-only", action="store_true",
                    help="time only the chunk-size sweep and print its JSON object")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode step and print its JSON object")
    ap.add_argument("--ragged-only", action="store_true",
                    help="time only the ragged (serving-form) decode step and print its JSON object")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward pass and print its JSON object")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 256 MiB device copy three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the STILL operator here runs on a single MI355X "
              f"(no sharding or collectives are built); --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from hybrid_sparse_softmax_amd import still
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    still.lib()
    if args.calibrate_copy:
        nbytes = 256 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}),
              flush=True)
        return
    if args.decode_only:
        print(json.dumps(bench_decode(still, torch, args.decode_steps, args.warmup)), flush=True)
        return
    if args.backward_only:
        print(json.dumps(bench_backward(still, torch, args.steps, args.warmup)), flush=True)
        return
    if args.chunk_sweep_only:
        print(json.dumps(bench_chunk_sweep(still, torch)), flush=True)
        return
    if args.ragged_only:
        print(json.dumps(bench_decode_ragged(still, torch, args.decode_steps, args.warmup)), flush=True)
        return
    pre = bench_prefill(still, torch, args.workload, args.steps, args.warmup)
    cfg = pre["cfg"]
    dec = None if args.no_decode else bench_decode(still, torch, args.decode_steps, args.warmup)
    dec_r = None if args.no_decode else bench_decode_ragged(still, torch, args.decode_steps,
                                                             args.warmup)
    bwd = None if args.no_backward else bench_backward(still, torch, max(3, args.steps // 4),
                                                         args.warmup)
    util = None if args.no_utility else bench_utility(still, torch)
    nsc = None if args.no_scaling else bench_n_scaling(still, torch)
    csw = None if args.no_chunk_sweep else bench_chunk_sweep(still, torch)
    cpu = None if args.no_cpu else cpu_baseline(pre["raw"], cfg)
    tok_s = pre["tokens"] / (pre["ms"] * 1e-3)
    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: batch {cfg['batch']}, seq {cfg['seqlen']}, "
                               f"{cfg['n_q_heads']} q / {cfg['n_kv_heads']} KV heads, d {cfg['head_dim']}, "
                               f"window {cfg['window']}, chunk {cfg['chunk']}, top-{cfg['topk']} per chunk",
                   "batch": cfg["batch"], "seq_len": cfg["seqlen"]},
        "roofline": pre["roof"],
        "cpu_baseline": cpu,
        "whole_step_TFLOPs": round(pre["total_alg"] / (pre["ms"] * 1e-3) / 1e12, 2),
        "kernels_ms": {k: round(v, 4) for k, v in pre["kern"].items()},
        "decode": dec,
        "decode_ragged": dec_r,
        "backward": bwd,
        "future_kv_utility": util,
        "n_scaling": nsc,
        "chunk_sweep": csw,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
