"""Pins of the oracle's gate (reading R-GATE: gamma = sigmoid(g) weighs the
linear branch inside the shared normaliser) against facts the oracle does
not compute itself: scipy's logistic function, torch's SDPA with an explicit
mask (gate closed: window + selected softmax attention), the ungated
operator (gate open), the odds law that placing gamma inside the shared
normaliser implies, the recurrent form, and finite differences for the
gate's gradient.  All CPU, float64."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O


def rand_inputs(seed, B, N, Hq, Hkv, d, scale_k=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d)) * scale_k
    v = rng.standard_normal((B, N, Hkv, d))
    wq = rng.standard_normal((Hkv, d // 2, d)) / math.sqrt(d)
    wk = rng.standard_normal((Hkv, d // 2, d)) / math.sqrt(d)
    gate = 2.0 * rng.standard_normal((B, N, Hq))
    dout = rng.standard_normal((B, N, Hq, d))
    return q, k, v, wq, wk, gate, dout


def test_gate_weight_is_the_logistic_function():
    x = np.concatenate([np.linspace(-40, 40, 801), [-1e4, 1e4, -745.0, 745.0]])
    np.testing.assert_allclose(O.gate_weight(x), scipy.special.expit(x), rtol=4e-15, atol=1e-300)
    assert O.gate_weight(0.0) == 0.5
    assert abs(O.gate_weight(math.log(3.0)) - 0.75) < 1e-16
    assert O.gate_weight(-np.inf) == 0.0 and O.gate_weight(np.inf) == 1.0
    np.testing.assert_allclose(O.gate_weight(x) + O.gate_weight(-x), 1.0, rtol=1e-15)


HYBRID = O.Params(window=4, chunk=4, topk=1)     # window + selected + linear


def sa_mask(route, N, W):
    """[N, N] bool: key j is a softmax key of query t (window or selected
    routed), written from the routing rule directly."""
    m = np.zeros((N, N), bool)
    for t in range(N):
        for j in range(t + 1):
            m[t, j] = j > t - W or route[j] == O.ROUTE_SA
    return m


def test_open_gate_is_the_ungated_operator():
    q, k, v, wq, wk, _, _ = rand_inputs(1, 2, 23, 4, 2, 8, scale_k=1.5)
    ref = O.fwd_direct(q, k, v, wq, wk, HYBRID)["out"]
    got = O.fwd_direct(q, k, v, wq, wk, HYBRID, gate=np.full((2, 23, 4), 50.0))["out"]
    np.testing.assert_array_equal(got, ref)


def test_closed_gate_is_window_plus_selected_softmax():
    """gamma = 0: the linear branch drops out and what remains is softmax
    attention over the window and the selected routed tokens (torch SDPA with
    that boolean mask, float64)."""
    q, k, v, wq, wk, _, _ = rand_inputs(2, 1, 27, 4, 2, 8, scale_k=1.5)
    o = O.fwd_direct(q, k, v, wq, wk, HYBRID, gate=np.full((1, 27, 4), -np.inf))
    for g in range(2):
        mask = torch.from_numpy(sa_mask(o["route"][0, g], 27, HYBRID.window))
        for h in (2 * g, 2 * g + 1):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[0, :, h])[None], torch.from_numpy(k[0, :, g])[None],
                torch.from_numpy(v[0, :, g])[None], attn_mask=mask[None])[0].numpy()
            np.testing.assert_allclose(o["out"][0, :, h], ref, rtol=1e-12, atol=1e-13)


def test_gate_scales_the_odds_of_the_linear_branch():
    """With gamma inside the shared normaliser, out(gamma) lies on the segment
    from the softmax-only output (gate closed) to the linear-only output
    (normalised phi weights over the linear tokens), and its odds
    w / (1 - w) of the linear end are gamma times the ungated ones.  A gate
    applied anywhere else (outside the normaliser, on the softmax branch)
    breaks this."""
    q, k, v, wq, wk, gate, _ = rand_inputs(3, 1, 26, 2, 1, 8, scale_k=1.5)
    gam = O.gate_weight(gate)
    o1 = O.fwd_direct(q, k, v, wq, wk, HYBRID)
    og = O.fwd_direct(q, k, v, wq, wk, HYBRID, gate=gate)["out"]
    o0 = O.fwd_direct(q, k, v, wq, wk, HYBRID, gate=np.full(gate.shape, -np.inf))["out"]
    route = o1["route"][0, 0]
    fk = O.np_map(k[0, :, 0], wk[0])
    checked = 0
    for t in range(26):
        la = [j for j in range(t - HYBRID.window + 1) if route[j] == O.ROUTE_LA]
        for h in range(2):
            if not la:
                np.testing.assert_allclose(og[0, t, h], o0[0, t, h], rtol=1e-13)
                continue
            kap = fk[la] @ O.np_map(q[0, t, h], wq[0])
            o_la = kap @ v[0, la, 0] / kap.sum()
            seg = o_la - o0[0, t, h]
            w1 = (o1["out"][0, t, h] - o0[0, t, h]) @ seg / (seg @ seg)
            np.testing.assert_allclose(o1["out"][0, t, h], o0[0, t, h] + w1 * seg, atol=1e-12)
            odds = gam[0, t, h] * w1 / (1.0 - w1)
            wg = odds / (1.0 + odds)
            np.testing.assert_allclose(og[0, t, h], o0[0, t, h] + wg * seg, rtol=1e-11, atol=1e-12)
            checked += 1
    assert checked > 20


def test_gated_direct_equals_recurrent():
    q, k, v, wq, wk, gate, _ = rand_inputs(4, 2, 30, 4, 2, 8, scale_k=1.5)
    for p in (HYBRID, O.Params(window=6, chunk=4, topk=2), O.Params(window=0, chunk=4, topk=0)):
        d = O.fwd_direct(q, k, v, wq, wk, p, gate=gate)["out"]
        r, _ = O.fwd_recurrent(q, k, v, wq, wk, p, gate=gate)
        np.testing.assert_allclose(d, r, rtol=1e-11, atol=1e-12)


def central_difference(f, x, h=1e-6):
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


@pytest.mark.parametrize("W,C,lam", [(4, 4, 2), (0, 4, 0), (6, 4, 1)])
def test_gated_bwd_matches_finite_differences(W, C, lam):
    """Every gradient of the gated operator, the gate logits' included, equals
    central differences of the gated forward (routing held fixed)."""
    q, k, v, wq, wk, gate, dout = rand_inputs(5 + W, 1, 13, 2, 1, 4, scale_k=1.5)
    p = O.Params(window=W, chunk=C, topk=lam)
    sel = O.fwd_direct(q, k, v, wq, wk, p)["sel_idx"] if lam > 0 else None
    zero_scores = np.zeros((1, 1, 13))

    def loss():
        out = O.fwd_direct(q, k, v, wq, wk, p, sel_override=sel, scores=zero_scores, gate=gate)["out"]
        return float((out * dout).sum())

    g = O.bwd_direct(q, k, v, wq, wk, dout, p, sel_idx=sel, gate=gate)
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dwq", wq), ("dwk", wk), ("dgate", gate)):
        fd = central_difference(loss, x)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(fd).max()),
                                   err_msg=name)
    rows = [(0, 0), (0, 7), (0, 12)]
    part = O.bwd_direct(q, k, v, wq, wk, dout, p, sel_idx=sel, gate=gate, rows=rows)
    for b, t in rows:
        np.testing.assert_allclose(part["dgate"][b, t], g["dgate"][b, t], rtol=1e-13, atol=1e-15)


def test_ungated_bwd_has_no_gate_gradient_and_open_gate_matches():
    q, k, v, wq, wk, _, dout = rand_inputs(7, 1, 15, 2, 1, 4, scale_k=1.5)
    g0 = O.bwd_direct(q, k, v, wq, wk, dout, HYBRID)
    g1 = O.bwd_direct(q, k, v, wq, wk, dout, HYBRID, gate=np.full((1, 15, 2), 50.0))
    assert "dgate" not in g0
    for name in ("dq", "dk", "dv", "dwq", "dwk"):
        np.testing.assert_array_equal(g1[name], g0[name])
    assert np.all(g1["dgate"] == 0)   # gamma (1 - gamma) = 0 at gamma = 1
