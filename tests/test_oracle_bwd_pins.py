"""Pins of the oracle's backward pass against what fixes a gradient without
the oracle's own chain rule: central finite differences of the pinned
forward (fwd_direct with the routing held fixed), and torch autograd through
its scaled-dot-product attention where the operator reduces to causal
softmax.  All CPU, float64."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def rand_inputs(seed, B, N, Hq, Hkv, d, scale_k=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d)) * scale_k
    v = rng.standard_normal((B, N, Hkv, d))
    wq = rng.standard_normal((Hkv, d // 2, d)) / math.sqrt(d)
    wk = rng.standard_normal((Hkv, d // 2, d)) / math.sqrt(d)
    dout = rng.standard_normal((B, N, Hq, d))
    return q, k, v, wq, wk, dout


def central_difference(f, x, h=1e-6):
    """d f / d x for a scalar f of the array x, element by element."""
    g = np.zeros_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        x0 = flat[i]
        flat[i] = x0 + h
        fp = f()
        flat[i] = x0 - h
        fm = f()
        flat[i] = x0
        gf[i] = (fp - fm) / (2 * h)
    return g


def test_np_map_vjp_matches_finite_differences():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 6))
    P = rng.standard_normal((4, 6)) / math.sqrt(6)
    dphi = rng.standard_normal((3, 8))
    loss = lambda: float((O.np_map(x, P) * dphi).sum())
    dx, dP = O.np_map_vjp(x, P, dphi)
    np.testing.assert_allclose(dx, central_difference(loss, x), rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(dP, central_difference(loss, P), rtol=1e-7, atol=1e-8)


def test_np_map_vjp_norm_direction_split():
    """phi depends on x's norm and on P x's direction only: scaling P by
    c > 0 leaves phi unchanged, so <dP, P> = 0; moving x along itself
    changes only the norm, so <dx, x> = <dz, z> (the norm's share)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(8)
    P = rng.standard_normal((4, 8))
    dphi = rng.standard_normal(8)
    dx, dP = O.np_map_vjp(x, P, dphi)
    assert abs((dP * P).sum()) < 1e-12 * max(1.0, np.abs(dP).max())
    # z = ||x|| uh is linear in ||x|| along x, and uh(P x) is scale-free, so
    # the derivative along x equals dz . z
    phi = O.np_map(x, P)
    h = 1e-6
    along = (O.np_map(x * (1 + h), P) - O.np_map(x * (1 - h), P)) @ dphi / (2 * h)
    assert abs(dx @ x - along) < 1e-7
    assert np.all(phi >= 0)


def test_np_map_vjp_zero_projection_is_zero():
    x = np.arange(1.0, 5.0)
    P = np.zeros((2, 4))
    dx, dP = O.np_map_vjp(x, P, np.ones(4))
    # with u = 0, z = 0 regardless of x: phi is flat there
    assert np.all(dP == 0)
    assert np.all(dx == 0)


CASES = [
    # (W, C, lam, N, Hq, Hkv)   ragged last chunk in every case
    (4, 4, 2, 13, 2, 1),        # window + selected + linear, GQA 2
    (4, 4, 0, 11, 2, 1),        # window + linear (no selection)
    (0, 4, 0, 9, 2, 1),         # linear only
    (6, 4, 1, 14, 2, 2),        # window longer than a chunk, two KV heads
]


@pytest.mark.parametrize("case", CASES)
def test_bwd_matches_finite_differences(case):
    W, C, lam, N, Hq, Hkv = case
    q, k, v, wq, wk, dout = rand_inputs(11 + N, 1, N, Hq, Hkv, 4, scale_k=1.5)
    p = O.Params(window=W, chunk=C, topk=lam)
    sel = O.fwd_direct(q, k, v, wq, wk, p)["sel_idx"] if lam > 0 else None
    zero_scores = np.zeros((1, Hkv, N))

    def loss():
        # the routing is a constant: pass the selection and skip rescoring
        out = O.fwd_direct(q, k, v, wq, wk, p, sel_override=sel, scores=zero_scores)["out"]
        return float((out * dout).sum())

    g = O.bwd_direct(q, k, v, wq, wk, dout, p, sel_idx=sel)
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dwq", wq), ("dwk", wk)):
        fd = central_difference(loss, x)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(fd).max()),
                                   err_msg=name)


def sdpa_grads(q, k, v, dout):
    """torch autograd through causal SDPA (float64, CPU), GQA by repeating
    KV heads; returns dq, dk, dv in [B, N, H, d] layout."""
    G = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).requires_grad_(True)
    tk = torch.from_numpy(k).requires_grad_(True)
    tv = torch.from_numpy(v).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(G, dim=1),
        tv.permute(0, 2, 1, 3).repeat_interleave(G, dim=1), is_causal=True)
    (o.permute(0, 2, 1, 3) * torch.from_numpy(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("W,C,lam", [(64, 8, 0), (8, 8, 8), (12, 4, 9)])
def test_bwd_causal_softmax_endpoints(W, C, lam):
    """Window covering the sequence, or every routed token selected: the
    operator is causal softmax, so its gradients are SDPA's and the NP-Map
    projections get none."""
    q, k, v, wq, wk, dout = rand_inputs(3, 2, 29, 4, 2, 8, scale_k=2.0)
    p = O.Params(window=W, chunk=C, topk=lam)
    g = O.bwd_direct(q, k, v, wq, wk, dout, p)
    dq, dk, dv = sdpa_grads(q, k, v, dout)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(g[name], ref, rtol=1e-10, atol=1e-11, err_msg=name)
    assert np.all(g["dwq"] == 0) and np.all(g["dwk"] == 0)


def test_bwd_pure_linear_attention_values_gradient():
    """W = 0, lambda = 0: out_t = sum_{j<=t} kappa_tj v_j / sum_{j<=t} kappa_tj,
    linear in v; its gradient w.r.t. v_j is sum_{t>=j} kappa_tj / den_t dout_t,
    computed here from the explicit matrix of weights."""
    q, k, v, wq, wk, dout = rand_inputs(4, 1, 10, 1, 1, 6)
    p = O.Params(window=0, chunk=4, topk=0)
    fq = O.np_map(q[0, :, 0], wq[0])
    fk = O.np_map(k[0, :, 0], wk[0])
    A = np.tril(fq @ fk.T)
    A = A / A.sum(1, keepdims=True)
    g = O.bwd_direct(q, k, v, wq, wk, dout, p)
    np.testing.assert_allclose(g["dv"][0, :, 0], A.T @ dout[0, :, 0], rtol=1e-12, atol=1e-13)


def test_bwd_sampled_rows_equal_full_dq():
    """The sampled-rows mode (used for full-size parity) visits only the
    given queries; their dq must equal the full computation's."""
    q, k, v, wq, wk, dout = rand_inputs(9, 2, 21, 4, 2, 8, scale_k=1.5)
    p = O.Params(window=4, chunk=4, topk=2)
    full = O.bwd_direct(q, k, v, wq, wk, dout, p)
    rows = [(0, 0), (0, 7), (1, 12), (1, 20)]
    part = O.bwd_direct(q, k, v, wq, wk, dout, p, rows=rows)
    for b, t in rows:
        np.testing.assert_allclose(part["dq"][b, t], full["dq"][b, t], rtol=1e-13, atol=1e-14)
    assert np.isnan(part["dq"][0, 1]).all() and set(part) == {"dq"}


def test_bwd_sampled_keys_equal_full_dk_dv():
    """The sampled-keys mode (used for full-size parity of the key side)
    visits only the queries that can see the given keys; their dk and dv
    must equal the full computation's.  The keys cover a selected key, a
    linear key, a key still in its window at the end and the last token."""
    q, k, v, wq, wk, dout = rand_inputs(10, 2, 23, 4, 2, 8, scale_k=1.5)
    p = O.Params(window=4, chunk=4, topk=2)
    full = O.bwd_direct(q, k, v, wq, wk, dout, p)
    sel = O.select_chunks(O.window_scores(q, k, p, 2), p)[0]
    picked = int(sel[1, 0, 1, 0])                     # a selected key of chunk 1
    unpicked = [j for j in range(4, 8) if j not in set(sel[1, 1, 1].tolist())][0]
    keys = [(0, 1, 0), (1, 0, picked), (1, 1, unpicked), (0, 0, 20), (1, 1, 22)]
    part = O.bwd_direct(q, k, v, wq, wk, dout, p, keys=keys)
    assert set(part) == {"dk", "dv"}
    for b, g, j in keys:
        np.testing.assert_allclose(part["dk"][b, j, g], full["dk"][b, j, g], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(part["dv"][b, j, g], full["dv"][b, j, g], rtol=1e-12, atol=1e-13)
    assert np.isnan(part["dk"][0, 1, 0]).all() and np.isnan(part["dv"][1, 0, 1]).all()
