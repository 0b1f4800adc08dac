"""CPU oracle for the STILL intra-layer hybrid attention operator.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.
The product path (the HIP library and its Python binding) never touches it,
and this module imports nothing from the product.

Everything is plain float64 numpy, one obvious step at a time.  Sources are
the paper "STILL: Selecting Tokens for Intra-Layer Hybrid Attention to
Linearize LLMs" (Meng et al., 2026), as printed on its web pages:

* full text (paperpeel): Sec. 3.1 "Selecting Tokens by Self-Saliency Score",
  Sec. 3.2 "Norm-Preserved Feature Map", Sec. 3.3 ("Recurrent Form",
  "Chunk-Wise Parallel Form", "Complexity Analysis"), Appendix A.2 (the
  linear-attention state recurrence), A.3 (Lemma 1 and its Remark),
  A.4 (budget certification), A.7.5 (window spans one chunk);
* list view (thelatestinai): captions of Fig. 1 and Fig. 2.

The display equations of those pages were lost in extraction, so several
steps are readings of the prose.  Each reading is named where it is used:

R-SCORE   Self-Saliency of token t = the epsilon-smoothed divergence between
          token t's own local attention row ``a`` (over its window, itself
          included) and the leave-one-out row ``a~`` (the same logits with the
          self term removed, renormalised; a~_t = 0):
              Score_t = sum_j a_j * ln((a_j + eps) / (a~_j + eps)).
          (A.3 Lemma 1: rises with the diagonal probability as eps -> 0;
          Remark: at finite eps it re-ranks by the whole leave-one-out change.)
R-GQA     Under grouped-query attention the routing score of a KV head is the
          mean of its query heads' scores, summed in ascending head order
          (Sec. 3.3: routing is per head; the caches are per KV head).
R-SELECT  For every complete chunk, keep the top-lambda tokens by score;
          ties go to the lower position; -0 == +0; NaN ranks lowest.
R-DELAY   Chunk c is decided when its last token arrives; token j's route is
          used by every query t with j <= t - W (the token has left the
          window).  Needs W >= C whenever lambda > 0 (A.7.5: the window
          spans one chunk; Sec. 3.3 Recurrent Form: routing happens when a
          token leaves the window, per chunk).
R-NPMAP   phi(x) = [softmax(z); softmax(-z)] with u = P x and
          z = ||x|| u / ||u||  (z = 0 when u = 0): direction from the learned
          projection, pretrained norm re-injected before the softmax
          (Sec. 2 Hedgehog form; Sec. 3.2; abstract).
R-AGG     One shared normaliser: SA tokens weigh exp(tau q.k), LA tokens weigh
          phi_q(q).phi_k(k); out = sum w v / sum w  (Fig. 2 "hybrid
          aggregation"; Fig. 1: the context is kept without loss).
R-SCALE   tau = 1/sqrt(d) unless given.
R-GATE    The gate W_g (list view Table 9, module ablation; full text Sec. 4.1
          training strategy and App. A.6.1: a gating projection trained with
          the feature map, adapted by LoRA beside W_q, W_k, W_v, W_o) is taken
          as one weight per token and query head on the linear branch, inside
          the shared normaliser:  gamma_t,h = sigmoid(g_t,h), where the logit
          g = x W_g is a projection of the layer input computed outside the
          operator like q, k and v, and the linear weights become
          gamma * phi_q(q).phi_k(k).  No gate (None) is gamma = 1, the
          operator without the component; gamma = 0 leaves window + selected
          softmax attention.
R-ROUTE   The routing criteria the pages compare with Self-Saliency under the
          same routing and cache settings (full text Sec. 4 ablation, Table 7;
          list view Tab. 10-11): "diagonal" = the token's own weight a_tt in
          its window row; "qk" = its own logit tau q_t.k_t; both averaged over
          the group's query heads like the Self-Saliency.  "keynorm" = ||k_t||,
          "uniform" = lambda tokens evenly spaced in each chunk (offsets
          floor(i C / lambda)), "random" = lambda tokens drawn uniformly per
          chunk; these three do not depend on the queries, so the KV head's
          score is the value itself.  The random draw is a counter-based
          uniform: splitmix64 (Steele, Lea and Flood 2014, in Vigna's
          formulation) of the counter ((b * Hkv + g) << 32) | t, top 24 bits
          times 2^-24, so any implementation reproduces it exactly.
R-UTIL    The future-KV-utility diagnostic (full text App. A.7.4, Table 12):
          a remote key's utility is the total full causal attention weight
          that every query after its window (t >= j + W) gives it, summed
          over the group's query heads; the selected remote tokens are
          compared with as many eligible keys ranked by that utility.
R-BWD     Gradients (the backward pass the pages need for their two-stage
          linearization: Sec. 4.1 "Experimental Setups", training strategy;
          App. A.6.1, primary configuration) treat the routing as a
          constant mask: nothing flows through the scores or the top-lambda,
          and where the NP-Map projection P x is zero the map is taken as
          locally constant.

Parity unpinned: the pages fix neither the exact Self-Saliency formula
(R-SCORE), nor the exact NP-Map (R-NPMAP), nor the exact weighting of the two
branches (R-AGG), nor the gate's form (R-GATE).  The functions implementing them are pinned to closed
forms, invariants and the method's endpoints (causal softmax, causal linear
attention, Lemma 1), but the readings themselves are the contract.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# route flag values (same meaning as the cache's win_route bytes)
PENDING, ROUTE_SA, ROUTE_LA = 0, 1, 2


@dataclass(frozen=True)
class Params:
    window: int          # W
    chunk: int           # C
    topk: int            # lambda, per chunk
    eps: float = 1e-6    # Self-Saliency smoothing (A.3: "infinitesimally small")
    scale: float = 0.0   # tau; 0 -> 1/sqrt(d)
    route: str = "saliency"   # routing criterion (R-ROUTE)

    def tau(self, d: int) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(d)

    def topk_eff(self) -> int:
        return min(self.topk, self.chunk)


def validate(p: Params, n_q_heads: int, n_kv_heads: int, feat_dim: int) -> None:
    """Shape rules that follow from R-DELAY and the GQA layout."""
    if n_kv_heads <= 0 or n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    if p.window < 0 or p.chunk <= 0 or p.topk < 0:
        raise ValueError("window >= 0, chunk > 0, topk >= 0")
    if p.window == 0 and p.topk > 0:
        raise ValueError("no window means no scores, so topk must be 0")
    if p.topk > 0 and p.window < p.chunk:
        raise ValueError("delayed selection needs window >= chunk")
    if feat_dim % 2:
        raise ValueError("NP-Map feature dimension must be even")
    if p.route not in ROUTES:
        raise ValueError(f"unknown routing criterion {p.route}")


def topk_for_budget(m: int, window: int, chunk: int, n_max: int) -> int:
    """Certified per-chunk quota (A.4): lambda = floor((m - W) / ceil(N_max / C)),
    so that T_max * lambda <= m - W for every length up to N_max."""
    t_max = -(-n_max // chunk)
    return max(0, (m - window) // t_max)


# --------------------------------------------------------------------------
# NP-Map (Sec. 3.2; reading R-NPMAP)
# --------------------------------------------------------------------------
def np_map(x: np.ndarray, P: np.ndarray) -> np.ndarray:
    """phi(x) for x [..., d] and projection P [d'/2, d]  ->  [..., d']."""
    x = np.asarray(x, np.float64)
    u = x @ np.asarray(P, np.float64).T                       # direction source
    nu = np.linalg.norm(u, axis=-1, keepdims=True)
    nx = np.linalg.norm(x, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        z = np.where(nu > 0, nx * u / np.where(nu > 0, nu, 1.0), 0.0)
    return np.concatenate([_softmax(z), _softmax(-z)], axis=-1)


def _softmax(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Self-Saliency (Sec. 3.1, A.3; reading R-SCORE)
# --------------------------------------------------------------------------
def self_saliency(logits: np.ndarray, diag: np.ndarray, eps: float) -> np.ndarray:
    """Score of each row of ``logits`` [R, K] whose own (diagonal) entry sits
    in column ``diag[r]``.  Masked-out keys carry -inf and contribute 0.

    a  = softmax over the row (the token's local attention row),
    a~ = softmax over the row with the diagonal removed (a~_diag = 0),
    Score = sum_j a_j * ln((a_j + eps) / (a~_j + eps)).
    """
    s = np.asarray(logits, np.float64)
    R = s.shape[0]
    rows = np.arange(R)
    a = _masked_softmax(s)
    s_loo = s.copy()
    s_loo[rows, diag] = -np.inf
    a_loo = _masked_softmax(s_loo)
    term = a * (np.log(a + eps) - np.log(a_loo + eps))
    return term.sum(axis=1)


ROUTES = ("saliency", "diagonal", "qk", "keynorm", "uniform", "random")
QUERY_FREE_ROUTES = ("keynorm", "uniform", "random")


def splitmix64(x: int) -> int:
    """One output of the splitmix64 generator for state x (R-ROUTE)."""
    m = (1 << 64) - 1
    z = (x + 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def random_score(b: int, g: int, t: int, n_kv_heads: int) -> float:
    """Uniform draw in [0, 1) of token t of (sequence b, KV head g)."""
    return (splitmix64(((b * n_kv_heads + g) << 32) | t) >> 40) * 2.0 ** -24


def query_free_score(route: str, k_t: np.ndarray, t: int, b: int, g: int, n_kv_heads: int,
                     p: Params) -> float:
    """Score of token t under a criterion that ignores the queries."""
    if route == "keynorm":
        return float(np.linalg.norm(np.asarray(k_t, np.float64)))
    if route == "uniform":
        C, lam = p.chunk, p.topk_eff()
        return 1.0 if (t % C) in {(i * C) // lam for i in range(lam)} else 0.0
    if route == "random":
        return random_score(b, g, t, n_kv_heads)
    raise ValueError(route)


def head_score(route: str, logits: np.ndarray, diag: np.ndarray, eps: float) -> np.ndarray:
    """Per-query-head routing score of each row of window logits (R-SCORE,
    R-ROUTE): Self-Saliency, the diagonal weight, or the own logit."""
    if route == "saliency":
        return self_saliency(logits, diag, eps)
    rows = np.arange(logits.shape[0])
    if route == "diagonal":
        return _masked_softmax(np.asarray(logits, np.float64))[rows, diag]
    if route == "qk":
        return np.asarray(logits, np.float64)[rows, diag]
    raise ValueError(route)


def _masked_softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax where -inf entries get weight 0; an all -inf row gives 0."""
    finite = np.isfinite(s)
    mx = np.where(finite, s, -np.inf).max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.where(finite, np.exp(np.where(finite, s, 0.0) - mx), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    return np.where(tot > 0, e / np.where(tot > 0, tot, 1.0), 0.0)


def window_scores(q: np.ndarray, k: np.ndarray, p: Params, n_kv_heads: int,
                  per_head: bool = False, block: int = 256) -> np.ndarray:
    """sigma[b, g, t]: Self-Saliency of every token, averaged over the query
    heads of KV head g (R-GQA).  The window of query t is
    J_t = [max(0, t-W+1), t].  With per_head=True returns [B, Hq, N] instead.

    Queries are taken in blocks only to bound memory; each row is still the
    plain definition over its own window."""
    B, N, Hq, d = q.shape
    W = p.window
    if W <= 0:
        raise ValueError("scores need a window")
    G = Hq // n_kv_heads
    tau = p.tau(d)
    if p.route in QUERY_FREE_ROUTES and not per_head:
        sig = np.zeros((B, n_kv_heads, N))
        for b in range(B):
            for g in range(n_kv_heads):
                for t in range(N):
                    sig[b, g, t] = query_free_score(p.route, k[b, t, g], t, b, g, n_kv_heads, p)
        return sig
    out = np.zeros((B, Hq, N))
    for b in range(B):
        for t0 in range(0, N, block):
            t1 = min(N, t0 + block)
            j0 = max(0, t0 - W + 1)
            keys = np.arange(j0, t1)
            ts = np.arange(t0, t1)
            # window mask: j in [t-W+1, t]
            mask = (keys[None, :] <= ts[:, None]) & (keys[None, :] > ts[:, None] - W)
            diag = ts - j0
            for h in range(Hq):
                g = h // G
                lg = tau * (q[b, t0:t1, h, :] @ k[b, j0:t1, g, :].T)
                lg = np.where(mask, lg, -np.inf)
                out[b, h, t0:t1] = head_score(p.route, lg, diag, p.eps)
    if per_head:
        return out
    sig = np.zeros((B, n_kv_heads, N))
    for g in range(n_kv_heads):
        acc = np.zeros((B, N))
        for h in range(g * G, (g + 1) * G):      # ascending head order
            acc = acc + out[:, h, :]
        sig[:, g, :] = acc / G
    return sig


# --------------------------------------------------------------------------
# Gate (R-GATE)
# --------------------------------------------------------------------------
def gate_weight(logits) -> np.ndarray:
    """gamma = sigmoid(g) = 1 / (1 + exp(-g)), evaluated without overflow:
    exp(g) / (1 + exp(g)) for g < 0.  g = -inf gives 0, g = +inf gives 1."""
    g = np.asarray(logits, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        pos = 1.0 / (1.0 + np.exp(-np.where(g >= 0, g, 0.0)))
        e = np.exp(np.where(g < 0, g, 0.0))
        neg = e / (1.0 + e)
    return np.where(g >= 0, pos, neg)


# --------------------------------------------------------------------------
# Per-chunk selection (Sec. 3.3 Chunk-Wise Parallel Form; R-SELECT)
# --------------------------------------------------------------------------
def rank_order(scores: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Indices that sort tokens best-first: higher score, then lower position.
    -0 is +0 (numpy compares them equal); NaN ranks below everything."""
    key = np.where(np.isnan(scores), -np.inf, scores)
    return np.lexsort((positions, -key))


def select_chunks(sigma: np.ndarray, p: Params, n_tokens: int | None = None):
    """Top-lambda per complete chunk.  sigma [B, Hkv, N].

    Returns (sel_idx [B, Hkv, n_full, lambda_eff] ascending positions,
             route [B, Hkv, N] in {PENDING, ROUTE_SA, ROUTE_LA}).
    Tokens of the last, incomplete chunk stay PENDING (R-DELAY)."""
    B, Hkv, N = sigma.shape
    C, lam = p.chunk, p.topk_eff()
    n_full = N // C
    sel = np.zeros((B, Hkv, n_full, lam), np.int64)
    route = np.full((B, Hkv, N), PENDING, np.uint8)
    for b in range(B):
        for g in range(Hkv):
            for c in range(n_full):
                pos = np.arange(c * C, (c + 1) * C)
                order = rank_order(sigma[b, g, pos], pos)
                chosen = np.sort(pos[order[:lam]])
                sel[b, g, c] = chosen
                route[b, g, pos] = ROUTE_LA
                route[b, g, chosen] = ROUTE_SA
    return sel, route


def route_from_selection(sel_idx: np.ndarray, N: int, C: int) -> np.ndarray:
    """Route flags implied by a given selection (used for the near-tie
    protocol, where the oracle is re-run with another selection)."""
    B, Hkv, n_full, _ = sel_idx.shape
    route = np.full((B, Hkv, N), PENDING, np.uint8)
    route[:, :, : n_full * C] = ROUTE_LA
    for b in range(B):
        for g in range(Hkv):
            route[b, g, sel_idx[b, g].reshape(-1)] = ROUTE_SA
    return route


# --------------------------------------------------------------------------
# Chunk-parallel forward, direct per-query form (Sec. 3.3; R-DELAY, R-AGG)
# --------------------------------------------------------------------------
def fwd_direct(q, k, v, wq, wk, p: Params, rows=None, sel_override=None, scores=None, gate=None):
    """Hybrid attention output from the explicit per-query index sets.

    q [B,N,Hq,d], k/v [B,N,Hkv,d], wq/wk [Hkv, d'/2, d]  (float64 views).
    rows: optional list of (b, t) to evaluate (default: every query).
    sel_override: optional sel_idx [B,Hkv,N//C,lambda] to route with instead
    of the oracle's own selection (near-tie protocol).
    scores: optional group scores [B,Hkv,N] already computed by window_scores
    (saves recomputing them when only a few rows are evaluated).
    gate: optional gate logits [B,N,Hq] (R-GATE); None is no gate.

    Returns dict(out [B,N,Hq,d] (NaN where not evaluated), scores, sel_idx, route,
    lse [B,N,Hq], has_linear [B,N,Hq]): lse is the log of the shared
    normaliser, ln(sum over SA_t of exp(tau q.k) + sum over LA_t of the
    gated linear weights), and has_linear whether LA_t carries any weight
    (list view Fig. 2, hybrid aggregation: one denominator for both kinds).

    For query t of head h (KV head g):
      J_t  = [max(0, t-W+1), t]                       window (softmax)
      R_t  = {j <= t-W}                               routed region
      SA_t = J_t  U  {j in R_t : route_j = SA}        exp(tau q.k) weights
      LA_t = R_t \\ SA_t                              gamma phi_q(q).phi_k(k) weights
      out  = sum_{SA_t u LA_t} w_j v_j / sum w_j
    """
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    validate(p, Hq, Hkv, 2 * wq.shape[1])
    G = Hq // Hkv
    W, tau = p.window, p.tau(d)

    if scores is not None:
        sigma = np.asarray(scores, np.float64)
    elif W > 0:
        sigma = window_scores(q, k, p, Hkv)
    else:
        sigma = np.zeros((B, Hkv, N))
    if p.topk_eff() > 0:
        sel_idx, route = select_chunks(sigma, p)
        if sel_override is not None:
            sel_idx = np.asarray(sel_override, np.int64)
            route = route_from_selection(sel_idx, N, p.chunk)
    else:
        sel_idx = np.zeros((B, Hkv, N // p.chunk, 0), np.int64)
        route = np.full((B, Hkv, N), ROUTE_LA, np.uint8)

    phik = np.stack([np_map(k[:, :, g, :], wk[g]) for g in range(Hkv)], axis=2)  # [B,N,Hkv,d']
    gam = np.ones((B, N, Hq)) if gate is None else gate_weight(gate)

    out = np.full(q.shape, np.nan)
    lse = np.full((B, N, Hq), np.nan)
    has_linear = np.zeros((B, N, Hq), bool)
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(N)]
    for b, t in rows:
        r_end = t - W + 1                       # R_t = [0, r_end)
        for g in range(Hkv):
            win = np.arange(max(0, t - W + 1), t + 1) if W > 0 else np.arange(0)
            routed = np.arange(0, max(0, r_end))
            if routed.size:
                rr = route[b, g, routed]
                if np.any(rr == PENDING):
                    raise AssertionError("a routed token has no decision")
                sa_routed = routed[rr == ROUTE_SA]
                la_routed = routed[rr == ROUTE_LA]
            else:
                sa_routed = la_routed = routed
            sa = np.concatenate([sa_routed, win])
            for h in range(g * G, (g + 1) * G):
                qv = q[b, t, h]
                s = tau * (k[b, sa, g, :] @ qv)
                w_la = phik[b, la_routed, g, :] @ np_map(qv, wq[g]) if la_routed.size else np.zeros(0)
                w_la = gam[b, t, h] * w_la
                # shared normaliser; subtracting M = max(0, max s) changes nothing
                M = max(0.0, s.max()) if s.size else 0.0
                w_sa = np.exp(s - M)
                w_la = w_la * math.exp(-M)
                num = w_sa @ v[b, sa, g, :] + (w_la @ v[b, la_routed, g, :] if la_routed.size else 0.0)
                den = w_sa.sum() + w_la.sum()
                out[b, t, h] = num / den
                lse[b, t, h] = M + math.log(den)
                has_linear[b, t, h] = bool(w_la.sum() > 0.0)
    return dict(out=out, scores=sigma, sel_idx=sel_idx, route=route, lse=lse, has_linear=has_linear)


# --------------------------------------------------------------------------
# Recurrent (decode) form (Sec. 3.3 Recurrent Form; A.2 state recurrence)
# --------------------------------------------------------------------------
def new_cache(B, Hkv, d, feat_dim, p: Params, cap: int) -> dict:
    """Empty decode cache, laid out like the library's cache tensors."""
    W, C = p.window, p.chunk
    return dict(
        win_k=np.zeros((B, Hkv, max(W, 1), d)), win_v=np.zeros((B, Hkv, max(W, 1), d)),
        win_route=np.zeros((B, Hkv, max(W, 1)), np.uint8),
        pend_score=np.zeros((B, Hkv, C)),
        sel_k=np.zeros((B, Hkv, cap, d)), sel_v=np.zeros((B, Hkv, cap, d)),
        sel_count=np.zeros((B, Hkv), np.int64),
        lin_S=np.zeros((B, Hkv, feat_dim, d)), lin_z=np.zeros((B, Hkv, feat_dim)),
        pos=0,
    )


def decode_step(cache: dict, q_t, k_t, v_t, wq, wk, p: Params, sel_override=None, gate_t=None):
    """One recurrent step at position t = cache['pos'] for every sequence.

    q_t [B,Hq,d], k_t/v_t [B,Hkv,d], gate_t: optional gate logits [B,Hq]
    (R-GATE).  Mutates the cache; returns out [B,Hq,d].

    Steps per (b, g):
      1. token j = t-W leaves the window: SA -> appended to the selected
         list (kept forever); LA -> S += phi_k(k_j) v_j^T, z += phi_k(k_j).
         With W = 0 the incoming token itself is that token.
      2. k_t, v_t enter the window ring at slot t mod W.
      3. Self-Saliency of t from its window row, mean over the group's
         heads -> pending score slot t mod C.
      4. Output over window + selected list (softmax weights) and the
         linear state (phi weights), one shared normaliser.
      5. If t closes its chunk, pick the chunk's top-lambda: those tokens
         are marked SA, the others LA.
    """
    q_t, k_t, v_t = (np.asarray(a, np.float64) for a in (q_t, k_t, v_t))
    B, Hq, d = q_t.shape
    Hkv = k_t.shape[1]
    G = Hq // Hkv
    W, C, lam = p.window, p.chunk, p.topk_eff()
    tau = p.tau(d)
    t = cache["pos"]
    gam = np.ones((B, Hq)) if gate_t is None else gate_weight(gate_t)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            # 1. eviction
            if W == 0:
                ev = (k_t[b, g], v_t[b, g], ROUTE_LA)
            elif t - W >= 0:
                slot = (t - W) % W
                r = ROUTE_LA if lam == 0 else cache["win_route"][b, g, slot]
                if r == PENDING:
                    raise AssertionError("token left the window before its chunk was decided")
                ev = (cache["win_k"][b, g, slot].copy(), cache["win_v"][b, g, slot].copy(), r)
            else:
                ev = None
            if ev is not None:
                kj, vj, r = ev
                if r == ROUTE_SA:
                    n = cache["sel_count"][b, g]
                    if n >= cache["sel_k"].shape[2]:
                        raise OverflowError("selected cache is full")
                    cache["sel_k"][b, g, n] = kj
                    cache["sel_v"][b, g, n] = vj
                    cache["sel_count"][b, g] = n + 1
                else:
                    f = np_map(kj, wk[g])
                    cache["lin_S"][b, g] += np.outer(f, vj)
                    cache["lin_z"][b, g] += f
            # 2. window write
            if W > 0:
                cache["win_k"][b, g, t % W] = k_t[b, g]
                cache["win_v"][b, g, t % W] = v_t[b, g]
                cache["win_route"][b, g, t % W] = PENDING
                win_pos = np.arange(max(0, t - W + 1), t + 1)
                slots = win_pos % W
                wk_ = cache["win_k"][b, g, slots]
                wv_ = cache["win_v"][b, g, slots]
            n = cache["sel_count"][b, g]
            sk, sv = cache["sel_k"][b, g, :n], cache["sel_v"][b, g, :n]
            score_sum = 0.0
            for h in range(g * G, (g + 1) * G):
                qv = q_t[b, h]
                if W > 0:
                    lw = tau * (wk_ @ qv)
                    if p.route not in QUERY_FREE_ROUTES:
                        score_sum += head_score(p.route, lw[None, :], np.array([len(lw) - 1]), p.eps)[0]
                    s = np.concatenate([tau * (sk @ qv), lw])
                    vv = np.concatenate([sv, wv_])
                else:
                    s = tau * (sk @ qv)
                    vv = sv
                fq = gam[b, h] * np_map(qv, wq[g])
                M = max(0.0, s.max()) if s.size else 0.0
                w_sa = np.exp(s - M)
                num = w_sa @ vv + math.exp(-M) * (fq @ cache["lin_S"][b, g])
                den = w_sa.sum() + math.exp(-M) * (fq @ cache["lin_z"][b, g])
                out[b, h] = num / den
            # 3. pending score
            if W > 0:
                cache["pend_score"][b, g, t % C] = (
                    query_free_score(p.route, k_t[b, g], t, b, g, Hkv, p)
                    if p.route in QUERY_FREE_ROUTES else score_sum / G)
            # 5. chunk end
            if W > 0 and t % C == C - 1:
                pos = np.arange(t - C + 1, t + 1)
                if lam > 0:
                    order = rank_order(cache["pend_score"][b, g, pos % C], pos)
                    chosen = set(pos[order[:lam]].tolist())
                else:
                    chosen = set()
                if sel_override is not None:
                    chosen = set(np.asarray(sel_override[b, g, t // C]).tolist())
                for j in pos:
                    cache["win_route"][b, g, j % W] = ROUTE_SA if j in chosen else ROUTE_LA
    cache["pos"] = t + 1
    return out


def fwd_recurrent(q, k, v, wq, wk, p: Params, cap: int | None = None, sel_override=None,
                  gate=None):
    """Run the recurrent form token by token from an empty cache (gate:
    optional logits [B,N,Hq]).  Returns (out [B,N,Hq,d], cache after N tokens)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    validate(p, Hq, Hkv, 2 * wq.shape[1])
    if cap is None:
        cap = p.topk_eff() * (-(-N // p.chunk)) + 1
    cache = new_cache(B, Hkv, d, 2 * wq.shape[1], p, cap)
    out = np.zeros(q.shape)
    for t in range(N):
        out[:, t] = decode_step(cache, q[:, t], k[:, t], v[:, t], wq, wk, p, sel_override,
                                None if gate is None else np.asarray(gate)[:, t])
    return out, cache


# --------------------------------------------------------------------------
# Backward pass (gradients of the chunk-parallel form with the routing held
# fixed).  R-BWD: the selection is a constant mask -- no gradient flows
# through the scores, the top-lambda or the route flags; M = max(0, max s)
# cancels between numerator and denominator, so it carries none either.
# The gradient is the chain rule of fwd_direct's formulas, written out per
# query; every step below is the derivative of one step there.
# --------------------------------------------------------------------------
def np_map_vjp(x, P, dphi):
    """Vector-Jacobian product of np_map at x [..., d] with projection P
    [d'/2, d]: returns (dx [..., d], dP [d'/2, d]) for the cotangent dphi
    [..., d'].  Where u = P x is zero the map is taken as locally constant
    (zero gradient): z is pinned to 0 there by R-NPMAP.

    Steps (reverse order of np_map):
      a = softmax(z), b = softmax(-z):
          dz = a * (da - <da, a>) - b * (db - <db, b>)
      z = ||x|| * uh with uh = u / ||u||:
          d||x|| = <dz, uh>,  duh = ||x|| dz
      uh = u / ||u||:   du = (duh - <duh, uh> uh) / ||u||
      ||x||:            dx = d||x|| * x / ||x||
      u = P x:          dx += P^T du,  dP = du x^T (summed over rows)"""
    x = np.asarray(x, np.float64)
    P = np.asarray(P, np.float64)
    dphi = np.asarray(dphi, np.float64)
    half = P.shape[0]
    u = x @ P.T
    nu = np.linalg.norm(u, axis=-1, keepdims=True)
    nx = np.linalg.norm(x, axis=-1, keepdims=True)
    ok = nu > 0
    uh = np.where(ok, u / np.where(ok, nu, 1.0), 0.0)
    z = nx * uh
    a, bm = _softmax(z), _softmax(-z)
    da, db = dphi[..., :half], dphi[..., half:]
    dz = a * (da - (da * a).sum(-1, keepdims=True)) - bm * (db - (db * bm).sum(-1, keepdims=True))
    dnx = (dz * uh).sum(-1, keepdims=True)
    duh = nx * dz
    du = np.where(ok, (duh - (duh * uh).sum(-1, keepdims=True) * uh) / np.where(ok, nu, 1.0), 0.0)
    dnx = np.where(ok, dnx, 0.0)
    dx = np.where(nx > 0, dnx * x / np.where(nx > 0, nx, 1.0), 0.0) + du @ P
    dP = du.reshape(-1, half).T @ x.reshape(-1, x.shape[-1])
    return dx, dP


def bwd_direct(q, k, v, wq, wk, dout, p: Params, sel_idx=None, rows=None, keys=None, gate=None):
    """Gradients of L = sum(dout * out) with out = fwd_direct(q, k, v, wq,
    wk, p) and the routing fixed to ``sel_idx`` [B, Hkv, N//C, lambda]
    (the forward's own selection when None).

    Returns dict(dq, dk, dv [shapes of q, k, v], dwq, dwk [shape of wq]), plus
    dgate [B, N, Hq] when gate logits [B, N, Hq] are given (R-GATE).
    rows: optional list of distinct (b, t); then only those queries are visited and
    only dq (and dgate) is returned (NaN elsewhere): dq of a query depends on
    that query alone, while every key-side gradient sums over all queries.
    keys: optional list of (b, g, j); then only the queries that can see key
    j of (b, g) are visited -- t >= j of the heads of KV head g -- and only
    dk and dv are returned, at those keys (NaN elsewhere).  A key's gradient
    sums over exactly those queries.

    Per query t of head h (KV head g), with the sets of fwd_direct:
      w_j = exp(s_j - M) on SA_t, gamma exp(-M) kappa_j on LA_t,
      kappa_j = phi_q . phi_k(k_j), gamma = sigmoid(gate) (1 without a gate)
      den = sum w_j,  out = sum w_j v_j / den,  Dt = dout . out
      SA:  ds_j = (w_j / den) (dout . v_j - Dt);  dq += tau ds_j k_j;
           dk_j += tau ds_j q;  dv_j += (w_j / den) dout
      LA:  dkappa_j = (gamma exp(-M) / den) (dout . v_j - Dt);
           dphi_q += dkappa_j phi_k(k_j);  dphi_k(k_j) += dkappa_j phi_q;
           dv_j += (w_j / den) dout
      gate: dgamma = sum over LA_t of (exp(-M) kappa_j / den) (dout . v_j - Dt),
           dgate = gamma (1 - gamma) dgamma
    then the NP-Map's vector-Jacobian product carries dphi_q to q and W_phi_q,
    dphi_k to k and W_phi_k."""
    q, k, v, dout = (np.asarray(a, np.float64) for a in (q, k, v, dout))
    wq, wk = np.asarray(wq, np.float64), np.asarray(wk, np.float64)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    validate(p, Hq, Hkv, 2 * wq.shape[1])
    G = Hq // Hkv
    W, tau = p.window, p.tau(d)
    if p.topk_eff() > 0:
        if sel_idx is None:
            sel_idx = select_chunks(window_scores(q, k, p, Hkv), p)[0]
        route = route_from_selection(np.asarray(sel_idx, np.int64), N, p.chunk)
    else:
        route = np.full((B, Hkv, N), ROUTE_LA, np.uint8)

    phik = np.stack([np_map(k[:, :, g, :], wk[g]) for g in range(Hkv)], axis=2)
    gam = np.ones((B, N, Hq)) if gate is None else gate_weight(gate)
    dgate = np.zeros((B, N, Hq))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dphiq = np.zeros(q.shape[:3] + (2 * wq.shape[1],))
    dphik = np.zeros_like(phik)
    groups = {b: range(Hkv) for b in range(B)}
    if keys is not None:
        keys = [tuple(int(x) for x in key) for key in keys]
        first = {}
        for b, g, j in keys:
            first[b] = min(first.get(b, N), j)
        visit = [(b, t) for b in sorted(first) for t in range(first[b], N)]
        groups = {b: sorted({g for bb, g, _ in keys if bb == b}) for b in first}
    elif rows is None:
        visit = [(b, t) for b in range(B) for t in range(N)]
    else:
        visit = list(rows)
    for b, t in visit:
        r_end = t - W + 1
        for g in groups[b]:
            win = np.arange(max(0, t - W + 1), t + 1) if W > 0 else np.arange(0)
            routed = np.arange(0, max(0, r_end))
            rr = route[b, g, routed]
            if np.any(rr == PENDING):
                raise AssertionError("a routed token has no decision")
            sa = np.concatenate([routed[rr == ROUTE_SA], win])
            la = routed[rr == ROUTE_LA]
            for h in range(g * G, (g + 1) * G):
                qv, do = q[b, t, h], dout[b, t, h]
                s = tau * (k[b, sa, g, :] @ qv)
                fq = np_map(qv, wq[g])
                kap = phik[b, la, g, :] @ fq
                M = max(0.0, s.max()) if s.size else 0.0
                w_sa = np.exp(s - M)
                gm = gam[b, t, h]
                w_la = gm * math.exp(-M) * kap
                den = w_sa.sum() + w_la.sum()
                o = (w_sa @ v[b, sa, g, :] + w_la @ v[b, la, g, :]) / den
                Dt = do @ o
                ds = (w_sa / den) * (v[b, sa, g, :] @ do - Dt)
                dq[b, t, h] += tau * (ds @ k[b, sa, g, :])
                np.add.at(dk[b, :, g, :], sa, tau * np.outer(ds, qv))
                np.add.at(dv[b, :, g, :], sa, np.outer(w_sa / den, do))
                vd_la = v[b, la, g, :] @ do - Dt
                dgate[b, t, h] = gm * (1.0 - gm) * ((math.exp(-M) / den) * (kap @ vd_la))
                dkap = (gm * math.exp(-M) / den) * vd_la
                dphiq[b, t, h] += dkap @ phik[b, la, g, :]
                np.add.at(dphik[b, :, g, :], la, np.outer(dkap, fq))
                np.add.at(dv[b, :, g, :], la, np.outer(w_la / den, do))
    if keys is not None:
        dk_keys, dv_keys = np.full(k.shape, np.nan), np.full(v.shape, np.nan)
        for b, g, j in keys:
            dx, _ = np_map_vjp(k[b, j, g], wk[g], dphik[b, j, g])
            dk_keys[b, j, g] = dk[b, j, g] + dx
            dv_keys[b, j, g] = dv[b, j, g]
        return dict(dk=dk_keys, dv=dv_keys)
    dgate_out = {} if gate is None else {"dgate": dgate}
    if rows is not None:
        dq_rows = np.full(q.shape, np.nan)
        for b, t in visit:
            for g in range(Hkv):
                for h in range(g * G, (g + 1) * G):
                    dx, _ = np_map_vjp(q[b, t, h], wq[g], dphiq[b, t, h])
                    dq_rows[b, t, h] = dq[b, t, h] + dx
        if gate is not None:
            dg_rows = np.full(dgate.shape, np.nan)
            for b, t in visit:
                dg_rows[b, t] = dgate[b, t]
            dgate_out = {"dgate": dg_rows}
        return dict(dq=dq_rows, **dgate_out)
    dwq, dwk = np.zeros_like(wq), np.zeros_like(wk)
    for g in range(Hkv):
        for h in range(g * G, (g + 1) * G):
            dx, dP = np_map_vjp(q[:, :, h, :], wq[g], dphiq[:, :, h, :])
            dq[:, :, h, :] += dx
            dwq[g] += dP
        dx, dP = np_map_vjp(k[:, :, g, :], wk[g], dphik[:, :, g, :])
        dk[:, :, g, :] += dx
        dwk[g] += dP
    return dict(dq=dq, dk=dk, dv=dv, dwq=dwq, dwk=dwk, **dgate_out)


# --------------------------------------------------------------------------
# Future KV utility (full text App. A.7.4, Table 12).  R-UTIL: a remote key
# j (one that has left the window of some later query, j <= N-1-W) is worth
# the total full-attention weight the queries after its window give it,
#     u[b, g, j] = sum over the query heads h of KV head g and the queries
#                  t >= j + W of softmax_j'(tau q_t,h . k_j'), j' <= t
# (full causal attention, nothing routed).  The diagnostic compares the
# routed-out tokens a criterion selected with the same number of eligible
# keys ranked by u (higher first, then lower position).
# --------------------------------------------------------------------------
def future_kv_utility(q, k, p: Params, n_kv_heads: int) -> np.ndarray:
    """u [B, Hkv, N] for q [B,N,Hq,d], k [B,N,Hkv,d] (float64)."""
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, N, Hq, d = q.shape
    G = Hq // n_kv_heads
    W, tau = p.window, p.tau(d)
    t = np.arange(N)
    causal = t[None, :] <= t[:, None]                 # [query t, key j]: j <= t
    remote = t[None, :] <= t[:, None] - W             # j <= t - W, i.e. t >= j + W
    u = np.zeros((B, n_kv_heads, N))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = tau * (q[b, :, h, :] @ k[b, :, g, :].T)
            a = _masked_softmax(np.where(causal, s, -np.inf))
            u[b, g] += np.where(remote, a, 0.0).sum(axis=0)
    return u


def kv_utility_overlap(sel_idx, util, N: int, W: int) -> np.ndarray:
    """[B, Hkv, 2]: (m, overlap) per (sequence, KV head): m = selected tokens
    that are eligible remote keys (j <= N-1-W), overlap = how many of them
    are among the top-m eligible keys by utility."""
    sel_idx = np.asarray(sel_idx, np.int64)
    B, Hkv = util.shape[:2]
    elig = np.arange(max(0, N - W))
    out = np.zeros((B, Hkv, 2), np.int64)
    for b in range(B):
        for g in range(Hkv):
            chosen = set(int(j) for j in sel_idx[b, g].reshape(-1) if 0 <= j < elig.size)
            m = len(chosen)
            order = rank_order(util[b, g, elig], elig)
            top = set(elig[order[:m]].tolist())
            out[b, g] = (m, len(chosen & top))
    return out
