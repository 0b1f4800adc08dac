"""float64 CPU oracle of the STILL hybrid attention operator.

Test infrastructure only: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are its only callers.  It shares no code
with the HIP library and imports nothing from it.
"""
from .still_oracle import (  # noqa: F401
    PENDING, ROUTE_SA, ROUTE_LA, Params, validate, topk_for_budget, np_map,
    self_saliency, window_scores, rank_order, select_chunks,
    route_from_selection, fwd_direct, new_cache, decode_step, fwd_recurrent,
    ROUTES, QUERY_FREE_ROUTES, splitmix64, random_score, query_free_score, head_score,
    np_map_vjp, bwd_direct, future_kv_utility, kv_utility_overlap, gate_weight,
)
