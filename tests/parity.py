"""Helpers shared by the GPU parity tests: input preparation (rounded once,
then handed to both sides), comparison metrics and the near-tie protocol for
selections.  No operator arithmetic lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
import workloads

BF16_TOL = 1e-2      # rel-L2 of the output, bf16 storage with fp32 accumulation
F32_TOL = 1e-5       # rel-L2 of the output, fp32 storage
TIE_TOL = 1e-6       # near-tie margin of the selection protocol
# Per-row bars: every output row (b, t, h) on its own, relative to its norm.
# A row's error is a few bf16 roundings of its d values (about 2^-9 each) or
# fp32 sums of the same terms as the oracle's, so these leave an order of
# magnitude while one wrong key, weight or row shows up far above them.
ROW_TOL_BF16 = 5e-2
ROW_TOL_F32 = 1e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def prepare(raw: dict, dtype: torch.dtype, device="cuda"):
    """Round q/k/v to the run's dtype once; return (device tensors, float64
    numpy views of the very same rounded values)."""
    dev, ref = {}, {}
    for key in ("q", "k", "v"):
        t = torch.from_numpy(raw[key]).to(dtype)
        ref[key] = t.to(torch.float64).numpy()
        dev[key] = t.to(device).contiguous()
    for key in ("wphi_q", "wphi_k"):
        t = torch.from_numpy(raw[key]).float()
        ref[key] = t.double().numpy()
        dev[key] = t.to(device).contiguous()
    return dev, ref


def make_case(name, B, N, Hq, Hkv, d, W, C, lam, dtype="bf16", seed=1, **knobs):
    cfg = dict(batch=B, seqlen=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C,
               topk=lam, dtype=dtype)
    cfg.update(knobs)
    return cfg


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_tol(dtype_name: str) -> float:
    return ROW_TOL_F32 if dtype_name == "f32" else ROW_TOL_BF16


def check_rows(got, want, tol: float, what: str = "out") -> float:
    """Every row (last axis) of got within tol of want, relative to the row's
    norm (floored at 1e-3 of the mean row norm, so that near-zero rows are
    judged against the tensor's scale).  Rows where want is NaN (not
    evaluated) are skipped.  Returns the worst row error; raises
    AssertionError naming the worst row otherwise."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    d = g.shape[-1]
    g2, w2 = g.reshape(-1, d), w.reshape(-1, d)
    ok = np.isfinite(w2).all(axis=1)
    if not ok.any():
        return 0.0
    norms = np.linalg.norm(w2[ok], axis=1)
    floor = 1e-3 * max(float(norms.mean()), 1e-300)
    err = np.linalg.norm(g2[ok] - w2[ok], axis=1) / np.maximum(norms, floor)
    err = np.where(np.isfinite(err), err, np.inf)
    i = int(np.argmax(err))
    worst = float(err[i])
    where = np.unravel_index(np.flatnonzero(ok)[i], g.shape[:-1])
    say(f"  {what}: worst row {tuple(int(x) for x in where)} rel err {worst:.3e} (bar {tol:g})")
    assert worst <= tol, f"{what}: row {tuple(int(x) for x in where)} off by {worst:.3e} > {tol:g}"
    return worst


def check_selection(gpu_sel: np.ndarray, sigma: np.ndarray, oracle_sel: np.ndarray, chunk: int,
                    tol: float = TIE_TOL):
    """Selections must match exactly, except where the swapped tokens' oracle
    scores lie within tol * max(1, |score|) of each other.  Returns
    (n_mismatched_chunks, worst_margin); raises AssertionError otherwise."""
    assert gpu_sel.shape == oracle_sel.shape, (gpu_sel.shape, oracle_sel.shape)
    bad = 0
    worst = 0.0
    diff = np.nonzero((np.sort(gpu_sel, -1) != oracle_sel).any(-1))
    for b, g, c in zip(*diff):
        gs, os_ = set(gpu_sel[b, g, c].tolist()), set(oracle_sel[b, g, c].tolist())
        assert len(gs) == len(gpu_sel[b, g, c]), f"duplicate picks in chunk {(b, g, c)}"
        assert all(c * chunk <= j < (c + 1) * chunk for j in gs), f"pick outside chunk {(b, g, c)}"
        only_gpu, only_orc = gs - os_, os_ - gs
        for i in only_gpu:
            for j in only_orc:
                si, sj = sigma[b, g, i], sigma[b, g, j]
                margin = abs(si - sj)
                worst = max(worst, margin)
                assert margin <= tol * max(1.0, abs(si), abs(sj)), (
                    f"selection differs beyond the near-tie margin at (b,g,c)={(b, g, c)}: "
                    f"gpu picks {i} ({si!r}), oracle picks {j} ({sj!r})")
        bad += 1
    return bad, worst


def sampled_rows(B, N, C, n_per_batch=24, seed=0, extra=()):
    """Query positions to evaluate one by one at sizes where the whole output
    is too slow for the oracle: the first and last tokens, chunk edges and
    random positions."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        ts = {0, 1, C - 1, C, 2 * C - 1, 2 * C, N - 1, N - 2, N // 2}
        ts |= set(rng.integers(0, N, size=n_per_batch).tolist())
        ts |= set(extra)
        rows += [(b, t) for t in sorted(ts) if 0 <= t < N]
    return rows
