"""Pins of the float64 oracle against facts it does not compute itself:
library routines (torch scaled-dot-product attention), closed forms of the
Self-Saliency definition, brute force, the NP-Map norm invariant, the paper's
budget rule (Appendix A.4) with the budgets its experiments state, and the
equivalence of the recurrent and chunk-parallel forms (Sec. 3.3).

All CPU; marked neither gpu nor slow."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(seed, B, N, Hq, Hkv, d, scale_k=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d)) * scale_k
    v = rng.standard_normal((B, N, Hkv, d))
    wq = rng.standard_normal((Hkv, d // 2, d)) / math.sqrt(d)
    wk = rng.standard_normal((Hkv, d // 2, d)) / math.sqrt(d)
    return q, k, v, wq, wk


def causal_softmax_attention(q, k, v):
    """torch's SDPA in float64 on the CPU, GQA by repeating KV heads."""
    B, N, Hq, d = q.shape
    G = Hq // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o.permute(0, 2, 1, 3).numpy()


# ---------------------------------------------------------------- P1, P2
@pytest.mark.parametrize("topk", [0, 3])
def test_window_covering_sequence_is_causal_softmax(topk):
    q, k, v, wq, wk = rand_inputs(1, 2, 37, 4, 2, 16)
    p = O.Params(window=64, chunk=8, topk=topk)
    res = O.fwd_direct(q, k, v, wq, wk, p)
    ref = causal_softmax_attention(q, k, v)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)
    # the shared normaliser is the causal softmax's: its log is the
    # logsumexp of tau q.k over j <= t (torch's, on the same float64 logits)
    B, N, Hq, d = q.shape
    for b in range(B):
        for h in range(Hq):
            s = torch.from_numpy(q[b, :, h] @ k[b, :, h // 2].T / math.sqrt(d))
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), -math.inf)
            np.testing.assert_allclose(res["lse"][b, :, h], torch.logsumexp(s, 1).numpy(), rtol=1e-12)
    assert not res["has_linear"].any()


@pytest.mark.parametrize("W,C,lam", [(8, 8, 8), (8, 8, 20), (12, 4, 4)])
def test_all_tokens_selected_is_causal_softmax(W, C, lam):
    """lambda >= C routes every token that leaves the window to SA, so each
    query sees all of its past through softmax: any gap or overlap between
    the window and the routed region would break this."""
    q, k, v, wq, wk = rand_inputs(2, 1, 45, 4, 1, 16, scale_k=2.0)
    p = O.Params(window=W, chunk=C, topk=lam)
    out = O.fwd_direct(q, k, v, wq, wk, p)["out"]
    np.testing.assert_allclose(out, causal_softmax_attention(q, k, v), rtol=1e-11, atol=1e-12)
    rec, _ = O.fwd_recurrent(q, k, v, wq, wk, p)
    np.testing.assert_allclose(rec, out, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P3
def test_no_window_is_causal_linear_attention():
    """W = 0, lambda = 0: out_t = sum_{j<=t} (phi_q.phi_k) v_j / sum (phi_q.phi_k),
    evaluated here as one masked matrix product in torch."""
    q, k, v, wq, wk = rand_inputs(3, 2, 40, 4, 2, 16)
    p = O.Params(window=0, chunk=8, topk=0)
    out = O.fwd_direct(q, k, v, wq, wk, p)["out"]
    rec, cache = O.fwd_recurrent(q, k, v, wq, wk, p)
    B, N, Hq, d = q.shape
    G = 2
    ref = np.zeros_like(out)
    mask = torch.tril(torch.ones(N, N, dtype=torch.float64))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            fq = torch.from_numpy(O.np_map(q[b, :, h], wq[g]))
            fk = torch.from_numpy(O.np_map(k[b, :, g], wk[g]))
            A = (fq @ fk.T) * mask
            ref[b, :, h] = ((A @ torch.from_numpy(v[b, :, g])) / A.sum(1, keepdim=True)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rec, ref, rtol=1e-12, atol=1e-13)
    # the recurrent state is the plain sum of phi_k(k_j) v_j^T over all tokens
    for b in range(B):
        for g in range(2):
            fk = O.np_map(k[b, :, g], wk[g])
            np.testing.assert_allclose(cache["lin_S"][b, g], fk.T @ v[b, :, g], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(cache["lin_z"][b, g], fk.sum(0), rtol=1e-12)


def test_uniform_feature_map_gives_shared_normaliser():
    """With P = 0 every phi is uniform, so each LA token weighs exactly 4/d'.
    The output must then be (sum_SA e^s v + 4/d' sum_LA v) / (sum_SA e^s + 4/d' |LA|)."""
    rng = np.random.default_rng(4)
    N, d, W, C, lam = 48, 8, 8, 8, 2
    q = rng.standard_normal((1, N, 1, d))
    k = rng.standard_normal((1, N, 1, d))
    v = rng.standard_normal((1, N, 1, d))
    z = np.zeros((1, d // 2, d))
    p = O.Params(window=W, chunk=C, topk=lam)
    res = O.fwd_direct(q, k, v, z, z, p)
    route = res["route"][0, 0]
    tau = 1 / math.sqrt(d)
    for t in range(N):
        sa = [j for j in range(t + 1) if j > t - W or route[j] == O.ROUTE_SA]
        la = [j for j in range(t + 1) if j not in sa]
        e = np.exp(tau * k[0, sa, 0] @ q[0, t, 0])
        wla = 4.0 / d
        num = e @ v[0, sa, 0] + wla * v[0, la, 0].sum(0)
        den = e.sum() + wla * len(la)
        np.testing.assert_allclose(res["out"][0, t, 0], num / den, rtol=1e-12)
        # the log of that shared denominator, and whether it has a linear part
        np.testing.assert_allclose(res["lse"][0, t, 0], math.log(den), rtol=1e-12)
        assert res["has_linear"][0, t, 0] == (len(la) > 0)


# ---------------------------------------------------------------- P4
def _brute_force_topk(scores, positions, lam):
    """The unique lam-subset whose every member beats every non-member
    (higher score, then lower position; NaN lowest; -0 == +0)."""
    key = [(-np.inf if np.isnan(s) else s) for s in scores]
    winners = []
    for sub in itertools.combinations(range(len(scores)), lam):
        rest = [i for i in range(len(scores)) if i not in sub]
        if all(key[a] > key[b] or (key[a] == key[b] and positions[a] < positions[b])
               for a in sub for b in rest):
            winners.append(sorted(positions[i] for i in sub))
    assert len(winners) == 1
    return winners[0]


def test_selection_matches_brute_force():
    rng = np.random.default_rng(5)
    C, lam = 8, 3
    for trial in range(200):
        s = rng.choice([0.0, -0.0, 0.5, 1.0, 1.5, np.nan, 2.0], size=C) if trial % 2 else rng.standard_normal(C)
        sigma = s[None, None, :].astype(np.float64)
        sel, route = O.select_chunks(sigma, O.Params(window=8, chunk=C, topk=lam))
        want = _brute_force_topk(list(s), list(range(C)), lam)
        assert sel[0, 0, 0].tolist() == want
        assert sorted(np.nonzero(route[0, 0] == O.ROUTE_SA)[0].tolist()) == want


def test_selection_counts_and_partial_chunk_stay_pending():
    rng = np.random.default_rng(6)
    N, C, lam = 100, 16, 5
    sigma = rng.standard_normal((2, 3, N))
    sel, route = O.select_chunks(sigma, O.Params(window=16, chunk=C, topk=lam))
    assert sel.shape == (2, 3, N // C, lam)
    assert (route[:, :, (N // C) * C:] == O.PENDING).all()
    assert ((route == O.ROUTE_SA).sum(-1) == lam * (N // C)).all()


# ---------------------------------------------------------------- P5
def test_np_map_norm_reinjection_closed_forms():
    """P = [I 0] keeps the first d/2 coordinates as the direction, but the
    magnitude must be ||x|| (all of x), not ||u||."""
    d = 8
    P = np.hstack([np.eye(d // 2), np.zeros((d // 2, d // 2))])
    x = np.zeros(d)
    x[0], x[d - 1] = 3.0, 4.0                      # ||x|| = 5, u = 3 e_1
    phi = O.np_map(x, P)
    n = d // 2
    assert phi[0] == pytest.approx(math.exp(5) / (math.exp(5) + n - 1), rel=1e-14)
    assert phi[1] == pytest.approx(1 / (math.exp(5) + n - 1), rel=1e-14)
    assert phi[n] == pytest.approx(math.exp(-5) / (math.exp(-5) + n - 1), rel=1e-14)
    assert phi[n + 1] == pytest.approx(1 / (math.exp(-5) + n - 1), rel=1e-14)
    # u = 0  ->  z = 0  ->  uniform halves
    y = np.zeros(d)
    y[d - 1] = 7.0
    np.testing.assert_allclose(O.np_map(y, P), np.full(d, 1 / n), rtol=1e-15)


def test_np_map_invariants():
    rng = np.random.default_rng(7)
    d = 16
    P = rng.standard_normal((d // 2, d))
    x = rng.standard_normal((50, d)) * rng.lognormal(0, 1, (50, 1))
    phi = O.np_map(x, P)
    assert (phi > 0).all()
    np.testing.assert_allclose(phi[:, : d // 2].sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(phi[:, d // 2:].sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(O.np_map(x, 3.7 * P), phi, rtol=1e-13)      # direction only
    # the logits recovered from phi have exactly the norm of x
    lp1, lp2 = np.log(phi[:, : d // 2]), np.log(phi[:, d // 2:])
    zdiff = (lp1 - lp2) / 2.0                         # z + const per row
    u = x @ P.T
    zhat = u / np.linalg.norm(u, axis=1, keepdims=True) * np.linalg.norm(x, axis=1, keepdims=True)
    np.testing.assert_allclose(zdiff - zdiff.mean(1, keepdims=True), zhat - zhat.mean(1, keepdims=True),
                               rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- P6
def test_score_single_token_window():
    eps = 1e-6
    s = O.self_saliency(np.array([[0.37]]), np.array([0]), eps)[0]
    assert s == pytest.approx(math.log(1 + 1 / eps), rel=1e-14)


@pytest.mark.parametrize("n", [2, 5, 64])
def test_score_uniform_row_closed_form(n):
    eps = 1e-6
    s = O.self_saliency(np.zeros((1, n)), np.array([n - 1]), eps)[0]
    want = (1 / n) * math.log((1 / n + eps) / eps) + ((n - 1) / n) * math.log((1 / n + eps) / (1 / (n - 1) + eps))
    assert s == pytest.approx(want, rel=1e-13)


def test_score_two_token_row_closed_form():
    eps = 1e-3
    for x in (-3.0, 0.0, 1.5):
        p = 1 / (1 + math.exp(-x))                 # diagonal probability
        s = O.self_saliency(np.array([[0.0, x]]), np.array([1]), eps)[0]
        want = (1 - p) * math.log((1 - p + eps) / (1 + eps)) + p * math.log((p + eps) / eps)
        assert s == pytest.approx(want, rel=1e-13)


def test_score_shift_invariant_and_masked_keys_ignored():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((6, 9))
    diag = np.full(6, 8)
    a = O.self_saliency(s, diag, 1e-6)
    np.testing.assert_allclose(O.self_saliency(s + 11.0, diag, 1e-6), a, rtol=1e-12)
    pad = np.concatenate([np.full((6, 3), -np.inf), s], axis=1)
    np.testing.assert_allclose(O.self_saliency(pad, diag + 3, 1e-6), a, rtol=1e-14)


def test_score_lemma1_monotone_in_diagonal_probability():
    """A.3 Lemma 1: with the off-diagonal logits fixed, the score rises
    strictly with the diagonal probability (here eps << p)."""
    rng = np.random.default_rng(9)
    ctx = rng.standard_normal(31)
    diag_logits = np.linspace(-4, 6, 60)
    rows = np.stack([np.append(ctx, x) for x in diag_logits])
    sc = O.self_saliency(rows, np.full(len(rows), 31), 1e-6)
    assert np.all(np.diff(sc) > 0)


def test_score_ranking_equals_diagonal_ranking_as_eps_vanishes():
    """Lemma 1 (eps -> 0+): ranking by score equals ranking by a_tt; the
    Remark: at a finite eps the two rankings can differ."""
    rng = np.random.default_rng(10)
    rows = rng.standard_normal((400, 16)) * 2.5
    diag = np.full(400, 15)
    a = np.exp(rows - rows.max(1, keepdims=True))
    p = a[:, 15] / a.sum(1)
    tiny = O.self_saliency(rows, diag, 1e-200)
    assert (np.argsort(tiny, kind="stable") == np.argsort(p, kind="stable")).all()
    big = O.self_saliency(rows, diag, 0.5)
    assert not (np.argsort(big, kind="stable") == np.argsort(p, kind="stable")).all()


def test_group_score_is_mean_of_head_scores():
    q, k, v, wq, wk = rand_inputs(11, 1, 30, 6, 2, 8)
    p = O.Params(window=8, chunk=8, topk=2)
    per_head = O.window_scores(q, k, p, 2, per_head=True)
    grp = O.window_scores(q, k, p, 2)
    np.testing.assert_allclose(grp[0, 0], per_head[0, 0:3].mean(0), rtol=1e-14)
    np.testing.assert_allclose(grp[0, 1], per_head[0, 3:6].mean(0), rtol=1e-14)


# ---------------------------------------------------------------- P7
CASES = [
    # B, N, Hq, Hkv, d, W, C, lam
    (1, 50, 2, 1, 8, 8, 8, 3),
    (2, 61, 4, 2, 16, 16, 8, 2),     # W > C, ragged tail
    (1, 40, 4, 4, 8, 8, 8, 0),       # SWA + LA only
    (1, 33, 2, 1, 8, 5, 8, 0),       # W < C allowed without selection
    (1, 30, 3, 1, 8, 0, 4, 0),       # pure linear
    (1, 70, 4, 1, 8, 16, 16, 16),    # everything routed to SA
]


@pytest.mark.parametrize("case", CASES)
def test_direct_equals_recurrent(case):
    B, N, Hq, Hkv, d, W, C, lam = case
    q, k, v, wq, wk = rand_inputs(12, B, N, Hq, Hkv, d, scale_k=1.5)
    p = O.Params(window=W, chunk=C, topk=lam)
    direct = O.fwd_direct(q, k, v, wq, wk, p)
    rec, cache = O.fwd_recurrent(q, k, v, wq, wk, p)
    np.testing.assert_allclose(rec, direct["out"], rtol=1e-10, atol=1e-12)
    # the recurrent form made the same decisions
    if W > 0:
        for b in range(B):
            for g in range(Hkv):
                for j in range(max(0, N - W), N):
                    r = cache["win_route"][b, g, j % W]
                    want = direct["route"][b, g, j] if lam > 0 else O.PENDING
                    if lam == 0 and j // C < N // C:
                        want = O.ROUTE_LA
                    assert r == want
    # every token that left the window as SA sits in the selected list
    n_left = max(0, N - W)                      # tokens j <= N-1-W
    want = int((direct["route"][0, 0, :n_left] == O.ROUTE_SA).sum()) if lam else 0
    assert cache["sel_count"][0, 0] == want


def test_prefill_then_decode_equals_longer_prefill():
    q, k, v, wq, wk = rand_inputs(13, 1, 75, 4, 2, 8, scale_k=1.5)
    p = O.Params(window=8, chunk=8, topk=3)
    full = O.fwd_direct(q, k, v, wq, wk, p)["out"]
    _, cache = O.fwd_recurrent(q[:, :50], k[:, :50], v[:, :50], wq, wk, p, cap=40)
    for t in range(50, 75):
        o = O.decode_step(cache, q[:, t], k[:, t], v[:, t], wq, wk, p)
        np.testing.assert_allclose(o, full[:, t], rtol=1e-10, atol=1e-12)


def test_selection_override_reproduces_own_selection():
    q, k, v, wq, wk = rand_inputs(14, 1, 64, 2, 1, 8)
    p = O.Params(window=8, chunk=8, topk=3)
    a = O.fwd_direct(q, k, v, wq, wk, p)
    b = O.fwd_direct(q, k, v, wq, wk, p, sel_override=a["sel_idx"])
    np.testing.assert_array_equal(a["out"], b["out"])
    other = a["sel_idx"].copy()
    other[0, 0, 3] = [24, 25, 26]
    c = O.fwd_direct(q, k, v, wq, wk, p, sel_override=other)
    assert not np.allclose(c["out"][0, 40:], a["out"][0, 40:])


# ---------------------------------------------------------------- P8, budget
def test_budget_helper_against_stated_budgets():
    with open(os.path.join(GOLDEN, "budgets.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        lam = O.topk_for_budget(c["m"], c["window"], c["chunk"], c["n_max"])
        assert lam == c["topk"], c
        t_max = -(-c["n_max"] // c["chunk"])
        assert t_max * lam <= c["m"] - c["window"] < t_max * (lam + 1)


def test_validation_rules():
    with pytest.raises(ValueError):
        O.validate(O.Params(window=0, chunk=8, topk=1), 4, 2, 8)
    with pytest.raises(ValueError):
        O.validate(O.Params(window=4, chunk=8, topk=1), 4, 2, 8)
    with pytest.raises(ValueError):
        O.validate(O.Params(window=8, chunk=8, topk=1), 3, 2, 8)
    O.validate(O.Params(window=4, chunk=8, topk=0), 4, 2, 8)


# ---------------------------------------------------------------- routing criteria (R-ROUTE)
def test_splitmix64_known_answers():
    """The published splitmix64 sequence started from state 0 (each call
    advances the state by the golden gamma before mixing)."""
    gamma = 0x9E3779B97F4A7C15
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [O.splitmix64((i * gamma) & ((1 << 64) - 1)) for i in range(3)]
    assert got == want


def test_random_route_is_uniform_and_reproducible():
    u = np.array([O.random_score(b, g, t, 8) for b in range(2) for g in range(8) for t in range(512)])
    assert ((u >= 0) & (u < 1)).all()
    assert abs(u.mean() - 0.5) < 0.01
    hist = np.histogram(u, bins=16, range=(0, 1))[0]
    assert hist.min() > 0.8 * len(u) / 16
    assert u[0] == O.random_score(0, 0, 0, 8)
    # every value is a multiple of 2^-24 (exact in fp32 as well)
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))


def test_query_free_routes_pick_by_their_definition():
    q, k, v, wq, wk = rand_inputs(21, 2, 70, 4, 2, 8)
    for route in ("keynorm", "uniform", "random"):
        p = O.Params(window=16, chunk=16, topk=3, route=route)
        sig = O.window_scores(q, k, p, 2)
        sel, _ = O.select_chunks(sig, p)
        for b in range(2):
            for g in range(2):
                for c in range(70 // 16):
                    pos = np.arange(16 * c, 16 * c + 16)
                    if route == "keynorm":
                        val = np.linalg.norm(k[b, pos, g], axis=1)
                    elif route == "uniform":
                        val = np.isin(pos % 16, [0, 5, 10]).astype(float)   # floor(16 i / 3)
                    else:
                        val = np.array([O.random_score(b, g, int(t), 2) for t in pos])
                    want = np.sort(pos[np.argsort(-val, kind="stable")[:3]])
                    np.testing.assert_array_equal(sel[b, g, c], want)


def test_diagonal_and_qk_routes_closed_forms():
    q, k, v, wq, wk = rand_inputs(22, 1, 20, 2, 1, 8)
    tau = 1 / math.sqrt(8)
    for route in ("diagonal", "qk"):
        p = O.Params(window=4, chunk=4, topk=1, route=route)
        sig = O.window_scores(q, k, p, 1)
        for t in range(20):
            vals = []
            for h in range(2):
                js = range(max(0, t - 3), t + 1)
                lg = np.array([tau * q[0, t, h] @ k[0, j, 0] for j in js])
                vals.append(math.exp(lg[-1]) / np.exp(lg).sum() if route == "diagonal" else lg[-1])
            assert abs(sig[0, 0, t] - (vals[0] + vals[1]) / 2) < 1e-12


@pytest.mark.parametrize("route", ["saliency", "diagonal"])
def test_window_scores_past_the_first_query_block(route):
    """window_scores evaluates queries in blocks (for memory); the rows of the
    blocks after the first (their key offset j0, the diagonal column and the
    window mask) must be each row's own window, scored on its own.  At
    N = 700 with blocks of 256 and 100 every row is compared with a
    brute-force per-row window: its logits written out one key at a time,
    the pinned single-row Self-Saliency (closed forms and Lemma 1 above) or
    the diagonal weight from explicit exponentials."""
    q, k, v, wq, wk = rand_inputs(24, 2, 700, 4, 2, 8, scale_k=1.5)
    W = 37
    p = O.Params(window=W, chunk=37, topk=1, route=route)
    tau = 1 / math.sqrt(8)
    per_head = {blk: O.window_scores(q, k, p, 2, per_head=True, block=blk) for blk in (256, 100)}
    sig = O.window_scores(q, k, p, 2)
    for b in range(2):
        for h in range(4):
            g = h // 2
            for t in range(700):
                js = range(max(0, t - W + 1), t + 1)
                lg = np.array([tau * float(q[b, t, h] @ k[b, j, g]) for j in js])
                if route == "saliency":
                    want = O.self_saliency(lg[None, :], np.array([len(lg) - 1]), p.eps)[0]
                else:
                    e = [math.exp(x - lg.max()) for x in lg]
                    want = e[-1] / sum(e)
                for blk, got in per_head.items():
                    assert abs(got[b, h, t] - want) <= 1e-12 * max(1.0, abs(want)), (blk, b, h, t)
    np.testing.assert_allclose(sig, per_head[256].reshape(2, 2, 2, 700).mean(axis=2), rtol=1e-13,
                               atol=1e-14)


def test_diagonal_route_ranks_like_saliency_as_eps_vanishes():
    """Lemma 1 again, through the whole selection: with eps -> 0 the
    Self-Saliency picks the same tokens as the diagonal weight."""
    q, k, v, wq, wk = rand_inputs(23, 1, 96, 2, 1, 8, scale_k=2.0)
    pd = O.Params(window=16, chunk=16, topk=4, route="diagonal")
    # per head the rankings agree (the group mean of two heads can re-rank),
    # so one query head per KV head
    q1, k1 = q[:, :, :1], k
    s1, _ = O.select_chunks(O.window_scores(q1, k1, O.Params(window=16, chunk=16, topk=4, eps=1e-200), 1),
                            O.Params(window=16, chunk=16, topk=4))
    s2, _ = O.select_chunks(O.window_scores(q1, k1, pd, 1), pd)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("route", ["diagonal", "qk", "keynorm", "uniform", "random"])
def test_direct_equals_recurrent_for_each_route(route):
    q, k, v, wq, wk = rand_inputs(24, 2, 45, 4, 2, 8, scale_k=1.5)
    p = O.Params(window=8, chunk=8, topk=3, route=route)
    direct = O.fwd_direct(q, k, v, wq, wk, p)
    rec, cache = O.fwd_recurrent(q, k, v, wq, wk, p)
    np.testing.assert_allclose(rec, direct["out"], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------- future KV utility (App. A.7.4)
def _sdpa_attention_matrix(q, k, h, g):
    """The full causal attention matrix of head h from torch's SDPA with the
    identity as values (out = A I = A), float64."""
    N, d = q.shape[1], q.shape[3]
    tq = torch.from_numpy(q[0, :, h, :])[None, None]
    tk = torch.from_numpy(k[0, :, g, :])[None, None]
    eye = torch.eye(N, dtype=torch.float64)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, eye, is_causal=True)[0, 0].numpy()


@pytest.mark.parametrize("W", [0, 4, 9])
def test_future_utility_against_sdpa_attention_matrix(W):
    q, k, v, wq, wk = rand_inputs(21, 1, 23, 4, 2, 8, scale_k=1.5)
    p = O.Params(window=W, chunk=4, topk=0)
    u = O.future_kv_utility(q, k, p, 2)
    t = np.arange(23)
    remote = t[None, :] <= t[:, None] - W
    for g in range(2):
        ref = sum(np.where(remote, _sdpa_attention_matrix(q, k, h, g), 0.0).sum(0) for h in (2 * g, 2 * g + 1))
        np.testing.assert_allclose(u[0, g], ref, rtol=1e-12, atol=1e-14)
    if W == 0:
        # every query row sums to one: the utilities of a KV head add up to G N
        np.testing.assert_allclose(u[0].sum(-1), 2 * 23, rtol=1e-12)
    else:
        # keys with no query after their window carry nothing
        assert np.all(u[0, :, 23 - W:] == 0)


def test_future_utility_two_tokens_closed_form():
    """N = 2, W = 1: only query 1 looks past key 0's window, so
    u[0] = e^{s10} / (e^{s10} + e^{s11}) and u[1] = 0."""
    q = np.array([[[[0.3, -1.2]], [[0.7, 0.4]]]])
    k = np.array([[[[1.0, 0.5]], [[-0.2, 0.9]]]])
    p = O.Params(window=1, chunk=1, topk=0)
    u = O.future_kv_utility(q, k, p, 1)
    tau = 1 / math.sqrt(2)
    s10, s11 = tau * q[0, 1, 0] @ k[0, 0, 0], tau * q[0, 1, 0] @ k[0, 1, 0]
    assert abs(u[0, 0, 0] - math.exp(s10) / (math.exp(s10) + math.exp(s11))) < 1e-15
    assert u[0, 0, 1] == 0.0


def test_utility_overlap_counts_by_brute_force():
    rng = np.random.default_rng(4)
    N, W = 40, 8
    util = rng.random((1, 1, N))
    sel = np.array([[[[3, 7], [9, 14], [17, 20], [25, 30], [33, 36]]]])  # 33, 36 are in the window region
    m, ov = O.kv_utility_overlap(sel, util, N, W)[0, 0]
    elig = list(range(N - W))
    chosen = {3, 7, 9, 14, 17, 20, 25, 30}
    top = sorted(elig, key=lambda j: (-util[0, 0, j], j))[:len(chosen)]
    assert m == 8 and ov == len(chosen & set(top))
    # selecting exactly the top keys gives full overlap
    sel2 = np.array(sorted(top)).reshape(1, 1, 4, 2)
    assert tuple(O.kv_utility_overlap(sel2, util, N, W)[0, 0]) == (8, 8)
