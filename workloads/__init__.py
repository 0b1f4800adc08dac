"""Seeded synthetic inputs for the STILL hybrid attention operator.

This module only draws random numbers in the shapes and distributions of the
workloads (Llama-3-8B-shaped attention layers, 32 query / 8 KV heads,
head_dim 128; the long-context setting of the paper's RULER experiments).  It
holds none of the operator's arithmetic, imports neither the oracle nor the
HIP library, and is the one piece of code both sides share.

Everything is drawn in float32 with numpy's PCG64 (``default_rng``); callers
round to the run's dtype (bf16 round-to-nearest-even via torch) and hand the
rounded values to both the GPU path and the oracle.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20260202

# name -> shape, parameters and value-distribution knobs.
CONFIGS: dict[str, dict] = {
    "toy_fp32": dict(index=1, batch=1, seqlen=256, n_q_heads=1, n_kv_heads=1, head_dim=64,
                     window=32, chunk=32, topk=8, dtype="f32",
                     n_heavy=4, heavy_scale=8.0),
    "prefill_4k": dict(index=2, batch=1, seqlen=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                       window=64, chunk=64, topk=16, dtype="bf16",
                       outlier_frac=0.01, heavy_scale=6.0),
    "prefill_16k": dict(index=3, batch=1, seqlen=16384, n_q_heads=32, n_kv_heads=8, head_dim=128,
                        window=64, chunk=64, topk=32, dtype="bf16",
                        outlier_frac=0.01, heavy_scale=6.0, needle=True),
    "train_8x2k": dict(index=4, batch=8, seqlen=2048, n_q_heads=32, n_kv_heads=8, head_dim=128,
                       window=64, chunk=64, topk=16, dtype="bf16"),
    "decode_b64_16k": dict(index=5, batch=64, pos=16384, n_q_heads=32, n_kv_heads=8, head_dim=128,
                           window=64, chunk=64, topk=32, dtype="bf16", sel_cap=8448),
}


def seed_of(name: str) -> int:
    return BASE_SEED + CONFIGS[name]["index"]


def shape_of(cfg: dict) -> dict:
    """The operator parameters of a config (no distribution knobs)."""
    keys = ("batch", "seqlen", "n_q_heads", "n_kv_heads", "head_dim", "window", "chunk", "topk", "dtype")
    return {k: cfg[k] for k in keys if k in cfg}


def make_prefill(cfg: dict, seed: int) -> dict:
    """q [B,N,Hq,d], k/v [B,N,Hkv,d], wphi_q/wphi_k [Hkv, d/2, d] (float32).

    Order of draws: q, k, v, per-token key-norm factors (lognormal(0, 0.5),
    shared by a token's KV heads), heavy/outlier positions (key scaled),
    the optional needle pair, the optional anti-aligned offsets (knob
    ``anti_align`` = a: queries + a u, keys - a u for a unit u per sequence
    and KV head, so every logit lies far below 0), then the NP-Map
    projections ~ N(0, 1/d)."""
    B, N = cfg["batch"], cfg["seqlen"]
    Hq, Hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    f = rng.lognormal(0.0, 0.5, size=(B, N)).astype(np.float32)
    k *= f[:, :, None, None]
    n_heavy = cfg.get("n_heavy", int(cfg.get("outlier_frac", 0.0) * N))
    if n_heavy:
        for b in range(B):
            pos = rng.choice(N, size=min(n_heavy, N), replace=False)
            k[b, pos] *= np.float32(cfg["heavy_scale"])
    needle = None
    if cfg.get("needle"):
        W = cfg["window"]
        needle = dict(key_pos=[], query_pos=N - 1)
        G = Hq // Hkv
        for b in range(B):
            p_key = int(rng.integers(0, max(1, N - 2 * W)))
            needle["key_pos"].append(p_key)
            for g in range(Hkv):
                u = rng.standard_normal(d)
                u /= np.linalg.norm(u)
                w = rng.standard_normal(d)
                w -= (w @ u) * u
                w /= np.linalg.norm(w)
                for h in range(g * G, (g + 1) * G):
                    q[b, N - 1, h] = np.linalg.norm(q[b, N - 1, h]) * u
                kn = np.linalg.norm(k[b, p_key, g])
                k[b, p_key, g] = kn * (0.9 * u + np.sqrt(0.19) * w)
    if cfg.get("anti_align"):
        # every query pushed along +a u_g and every key along -a u_g (one unit
        # direction per sequence and KV head): all logits sit far below 0
        a = np.float32(cfg["anti_align"])
        G = Hq // Hkv
        for b in range(B):
            for g in range(Hkv):
                u = rng.standard_normal(d)
                u = (u / np.linalg.norm(u)).astype(np.float32)
                q[b, :, g * G:(g + 1) * G] += a * u
                k[b, :, g] -= a * u
    sd = 1.0 / np.sqrt(d)
    wq = (rng.standard_normal((Hkv, d // 2, d)) * sd).astype(np.float32)
    wk = (rng.standard_normal((Hkv, d // 2, d)) * sd).astype(np.float32)
    return dict(q=q, k=k, v=v, wphi_q=wq, wphi_k=wk, needle=needle)


def make_grad_out(cfg: dict, seed: int) -> np.ndarray:
    """Upstream gradient of the output for the backward pass: dout
    [B, N, Hq, d] ~ N(0, 1), float32, from its own stream (seed + 1000003)
    so that it does not disturb the forward's draws."""
    rng = np.random.default_rng(seed + 1000003)
    return rng.standard_normal((cfg["batch"], cfg["seqlen"], cfg["n_q_heads"], cfg["head_dim"]),
                               dtype=np.float32)


def make_gate(cfg: dict, seed: int) -> np.ndarray:
    """Gate logits g [B, N, Hq] ~ N(0, 2^2), float32, from their own stream
    (seed + 2000003): gate weights sigmoid(g) spread over (0, 1)."""
    rng = np.random.default_rng(seed + 2000003)
    return (2.0 * rng.standard_normal((cfg["batch"], cfg["seqlen"], cfg["n_q_heads"]))).astype(np.float32)


def make_decode_stream(cfg: dict, seed: int, b: int, g: int) -> dict:
    """Cache contents of one (sequence, KV head) at position ``pos``:
    ring K/V of the last W tokens ~ N(0,1); route flags of the last complete
    chunk with ``topk`` seeded SA picks; n_sel = topk * floor((pos - W) / C)
    selected K/V rows ~ N(0,1); linear state S ~ N(0,1); normaliser z ~ |N(0,1)|
    (folded so the linear denominator stays positive)."""
    W, C, lam, d = cfg["window"], cfg["chunk"], cfg["topk"], cfg["head_dim"]
    pos = cfg["pos"]
    rng = np.random.default_rng([seed, b, g])
    win_k = rng.standard_normal((W, d), dtype=np.float32)
    win_v = rng.standard_normal((W, d), dtype=np.float32)
    # ring slot s holds position p with p % W == s; the chunk ending at pos-1
    # is complete, so its W (= C) tokens all carry a decision
    route = np.full(W, 2, np.uint8)
    picks = rng.permutation(W)[:lam]
    route[picks] = 1
    n_sel = lam * ((pos - W) // C)
    sel_k = rng.standard_normal((n_sel, d), dtype=np.float32)
    sel_v = rng.standard_normal((n_sel, d), dtype=np.float32)
    S = rng.standard_normal((d, d), dtype=np.float32)
    z = np.abs(rng.standard_normal(d, dtype=np.float32))
    return dict(win_k=win_k, win_v=win_v, win_route=route, sel_k=sel_k, sel_v=sel_v,
                sel_count=n_sel, lin_S=S, lin_z=z)


def make_decode_tokens(cfg: dict, seed: int, n_steps: int) -> dict:
    """New tokens for ``n_steps`` consecutive decode steps:
    q [K,B,Hq,d], k/v [K,B,Hkv,d] ~ N(0,1), plus the NP-Map projections."""
    B, Hq, Hkv, d = cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    rng = np.random.default_rng([seed, 1 << 20])
    q = rng.standard_normal((n_steps, B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((n_steps, B, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((n_steps, B, Hkv, d), dtype=np.float32)
    sd = 1.0 / np.sqrt(d)
    wq = (rng.standard_normal((Hkv, d // 2, d)) * sd).astype(np.float32)
    wk = (rng.standard_normal((Hkv, d // 2, d)) * sd).astype(np.float32)
    return dict(q=q, k=k, v=v, wphi_q=wq, wphi_k=wk)


def decode_positions(cfg: dict, seed: int) -> np.ndarray:
    """Per-sequence positions of a ragged decode batch (the serving mix):
    multiples of the chunk drawn uniformly from [1024, pos] (int64 [B])."""
    C = cfg["chunk"]
    rng = np.random.default_rng([seed, 1 << 21])
    return (C * rng.integers(1024 // C, cfg["pos"] // C + 1, size=cfg["batch"])).astype(np.int64)


def make_decode_cache(cfg: dict, seed: int, batches=None, positions=None) -> dict:
    """Whole-cache arrays in the library's cache layout for the sequences in
    ``batches`` (default: all), built from the per-stream draws of
    make_decode_stream; ``positions`` (per sequence, default cfg["pos"] for
    all) gives a ragged batch.  bf16 callers round sel/win K and V themselves."""
    B = cfg["batch"] if batches is None else len(batches)
    bs = list(range(cfg["batch"])) if batches is None else list(batches)
    Hkv, d, W, C, cap = cfg["n_kv_heads"], cfg["head_dim"], cfg["window"], cfg["chunk"], cfg["sel_cap"]
    out = dict(
        win_k=np.zeros((B, Hkv, W, d), np.float32), win_v=np.zeros((B, Hkv, W, d), np.float32),
        win_route=np.zeros((B, Hkv, W), np.uint8), pend_score=np.zeros((B, Hkv, C), np.float32),
        sel_k=np.zeros((B, Hkv, cap, d), np.float32), sel_v=np.zeros((B, Hkv, cap, d), np.float32),
        sel_count=np.zeros((B, Hkv), np.int32), lin_S=np.zeros((B, Hkv, d, d), np.float32),
        lin_z=np.zeros((B, Hkv, d), np.float32),
    )
    for i, b in enumerate(bs):
        for g in range(Hkv):
            s = make_decode_stream(cfg if positions is None else dict(cfg, pos=int(positions[b])),
                                   seed, b, g)
            n = s["sel_count"]
            out["win_k"][i, g] = s["win_k"]
            out["win_v"][i, g] = s["win_v"]
            out["win_route"][i, g] = s["win_route"]
            out["sel_k"][i, g, :n] = s["sel_k"]
            out["sel_v"][i, g, :n] = s["sel_v"]
            out["sel_count"][i, g] = n
            out["lin_S"][i, g] = s["lin_S"]
            out["lin_z"][i, g] = s["lin_z"]
    return out
