"""Host-side tests of the C ABI: the library loads, exports every entry point
include/still.h declares, sizes workspaces, and rejects every bad argument
with the documented status before launching anything (no GPU needed: all
of these calls return before the first HIP call)."""
import ctypes as ct
import json
import os
import re

import pytest

from hybrid_sparse_softmax_amd import still as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ct.c_void_p(0x1000)          # 16-byte aligned, never dereferenced
MISALIGNED = ct.c_void_p(0x1004)


def header_functions():
    txt = open(os.path.join(ROOT, "include", "still.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(still_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    L = S.lib()
    names = header_functions()
    assert set(names) == set(S.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert S.abi_version() == 6
    for code in (0, -1, -2, -3, -4, -5):
        assert S.status_str(code) and S.status_str(code) != "unknown status"
    assert S.status_str(7) == "unknown status"


def test_topk_for_budget_matches_stated_budgets():
    with open(os.path.join(ROOT, "tests", "golden", "budgets.json")) as f:
        for c in json.load(f)["cases"]:
            assert S.topk_for_budget(c["m"], c["window"], c["chunk"], c["n_max"]) == c["topk"]
    assert S.topk_for_budget(10, 64, 64, 100) == -1
    assert S.topk_for_budget(128, 64, 0, 100) == -1


def shape(**kw):
    base = dict(batch=1, seqlen=256, n_q_heads=4, n_kv_heads=2, head_dim=128, window=64,
                chunk=64, topk=16)
    base.update(kw)
    return S.make_shape(**base)


def fwd_status(sh, ws_bytes=1 << 40, cache=None, ptr=FAKE, ws=FAKE, gate=None, stats=None):
    return S.lib().still_hybrid_attn_fwd(ct.byref(sh), ptr, ptr, ptr, ptr, ptr, gate, ptr, None,
                                         None, stats, ct.byref(cache) if cache is not None else None, ws,
                                         ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=6, n_kv_heads=4), S.STILL_ERR_INVALID_ARG),      # G not integer
    (dict(window=0, topk=4), S.STILL_ERR_INVALID_ARG),                # no window, topk > 0
    (dict(window=32, chunk=64, topk=4), S.STILL_ERR_INVALID_ARG),     # W < C with selection
    (dict(chunk=0), S.STILL_ERR_INVALID_ARG),
    (dict(topk=-1), S.STILL_ERR_INVALID_ARG),
    (dict(seqlen=-5), S.STILL_ERR_INVALID_ARG),
    (dict(eps=0.0), S.STILL_ERR_INVALID_ARG),
    (dict(softmax_scale=-1.0), S.STILL_ERR_INVALID_ARG),
    (dict(head_dim=96), S.STILL_ERR_UNSUPPORTED),
    (dict(head_dim=128, feat_dim=64), S.STILL_ERR_UNSUPPORTED),
    (dict(n_q_heads=32, n_kv_heads=2), S.STILL_ERR_UNSUPPORTED),     # G = 16
])
def test_bad_shapes_rejected(kw, status):
    sh = shape(**kw)
    assert fwd_status(sh) == status
    n = ct.c_size_t(0)
    assert S.lib().still_fwd_workspace_size(ct.byref(sh), ct.byref(n)) == status
    assert S.lib().still_decode_workspace_size(ct.byref(sh), 64, ct.byref(n)) == status


def test_bad_dtype_and_flags():
    sh = shape()
    sh.dtype = 7
    assert fwd_status(sh) == S.STILL_ERR_INVALID_ARG
    sh = shape()
    sh.flags = 0x80
    assert fwd_status(sh) == S.STILL_ERR_INVALID_ARG
    # routing criteria 0-5 in bits 1-3; 6 and 7 are not defined
    for r in (6, 7):
        sh = shape()
        sh.flags = r << S.STILL_ROUTE_SHIFT
        assert fwd_status(sh) == S.STILL_ERR_INVALID_ARG
    for name in S.ROUTES:
        assert fwd_status(shape(route=name), ws_bytes=16) == S.STILL_ERR_WORKSPACE
    assert S.lib().still_fwd_workspace_size(None, ct.byref(ct.c_size_t())) == S.STILL_ERR_INVALID_ARG
    assert S.lib().still_fwd_workspace_size(ct.byref(shape()), None) == S.STILL_ERR_INVALID_ARG


def test_null_and_misaligned_pointers():
    sh = shape()
    assert fwd_status(sh, ptr=None) == S.STILL_ERR_INVALID_ARG
    assert fwd_status(sh, ptr=MISALIGNED) == S.STILL_ERR_INVALID_ARG
    assert fwd_status(sh, stats=MISALIGNED) == S.STILL_ERR_INVALID_ARG
    assert fwd_status(sh, stats=FAKE, ws_bytes=16) == S.STILL_ERR_WORKSPACE  # accepted, then too small


def test_workspace_size_and_too_small_workspace():
    sh = shape()
    need = S.fwd_workspace_size(sh)
    assert need > 0
    assert fwd_status(sh, ws_bytes=need - 1) == S.STILL_ERR_WORKSPACE
    assert fwd_status(sh, ws=None) == S.STILL_ERR_WORKSPACE
    # bigger problems need more
    assert S.fwd_workspace_size(shape(seqlen=4096)) > need
    assert S.decode_workspace_size(shape(), 8192) > S.decode_workspace_size(shape(), 64)


def test_empty_problems_are_noops():
    for kw in (dict(seqlen=0), dict(batch=0)):
        sh = shape(**kw)
        assert fwd_status(sh, ws_bytes=0, ws=None, ptr=None) == S.STILL_OK


def fake_cache(cap, pos, W=64, topk=16):
    c = S.CacheStruct(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, cap, 0x1000, 0x1000, pos)
    return c


def test_handoff_capacity_and_position_checks():
    sh = shape(seqlen=1024)                      # 16 selected per chunk
    need = 16 * ((1024 - 64 + 63) // 64)         # tokens that left the window
    assert fwd_status(sh, cache=fake_cache(need - 1, 1024)) == S.STILL_ERR_CAPACITY
    assert fwd_status(sh, cache=fake_cache(need, 1000)) == S.STILL_ERR_INVALID_ARG   # pos != N
    c = fake_cache(need, 1024)
    c.lin_S = None
    assert fwd_status(sh, cache=c) == S.STILL_ERR_INVALID_ARG
    # with enough capacity only the (fake) workspace size stops the call
    assert fwd_status(sh, cache=fake_cache(need, 1024), ws_bytes=16) == S.STILL_ERR_WORKSPACE


def decode_status(sh, cache, ws_bytes=1 << 40, ptr=FAKE, gate=None):
    return S.lib().still_hybrid_attn_decode_step(ct.byref(sh), ptr, ptr, ptr, ptr, ptr, gate,
                                                 ct.byref(cache), ptr, FAKE, ws_bytes, None)


def test_decode_capacity_guard():
    sh = shape(seqlen=1, topk=32)
    # step at t needs topk * ceil((t + 1 - W) / C) rows
    t = 16384
    need = 32 * ((t + 1 - 64 + 63) // 64)
    assert decode_status(sh, fake_cache(need - 1, t)) == S.STILL_ERR_CAPACITY
    assert decode_status(sh, fake_cache(need, t), ws_bytes=16) == S.STILL_ERR_WORKSPACE
    c = fake_cache(need, -1)
    assert decode_status(sh, c) == S.STILL_ERR_INVALID_ARG
    assert decode_status(sh, fake_cache(need, t), ptr=None) == S.STILL_ERR_INVALID_ARG


def test_decode_empty_batch_advances_position():
    sh = shape(seqlen=1, batch=0)
    c = fake_cache(64, 100)
    assert decode_status(sh, c, ws_bytes=0, ptr=None) == S.STILL_OK
    assert c.pos == 101


def ragged_status(sh, cache, pos_dev, max_pos, ws_bytes=1 << 40, ptr=FAKE):
    return S.lib().still_hybrid_attn_decode_step_ragged(ct.byref(sh), ptr, ptr, ptr, ptr, ptr, None,
                                                        ct.byref(cache), pos_dev, max_pos, ptr,
                                                        FAKE, ws_bytes, None)


def test_ragged_decode_checks():
    sh = shape(seqlen=1, topk=32)
    t = 16384
    need = 32 * ((t + 1 - 64 + 63) // 64)
    # capacity is checked against max_pos; cache.pos is not used (here -1)
    assert ragged_status(sh, fake_cache(need - 1, -1), FAKE, t) == S.STILL_ERR_CAPACITY
    assert ragged_status(sh, fake_cache(need, -1), FAKE, t, ws_bytes=16) == S.STILL_ERR_WORKSPACE
    assert ragged_status(sh, fake_cache(need, -1), None, t) == S.STILL_ERR_INVALID_ARG
    assert ragged_status(sh, fake_cache(need, -1), MISALIGNED, t) == S.STILL_ERR_INVALID_ARG
    assert ragged_status(sh, fake_cache(need, -1), FAKE, -1) == S.STILL_ERR_INVALID_ARG
    # an empty batch launches nothing and leaves cache.pos alone
    c = fake_cache(64, 7)
    assert ragged_status(shape(seqlen=1, batch=0), c, FAKE, 100, ws_bytes=0, ptr=None) == S.STILL_OK
    assert c.pos == 7


def bwd_status(sh, sel=FAKE, ws_bytes=1 << 40, ptr=FAKE, ws=FAKE, dw=FAKE, gate=None, dgate=None,
               out=None, stats=None, fws=None, fws_bytes=0):
    return S.lib().still_hybrid_attn_bwd(ct.byref(sh), ptr, ptr, ptr, ptr, ptr, gate, sel, ptr, out,
                                         stats, fws, fws_bytes, ptr, ptr, ptr, dw, dw, dgate, ws,
                                         ws_bytes, None)


def test_bwd_checks():
    sh = shape()
    need = S.bwd_workspace_size(sh)
    assert need > 0 and S.bwd_workspace_size(shape(seqlen=4096)) > need
    assert bwd_status(sh, ws_bytes=need - 1) == S.STILL_ERR_WORKSPACE
    assert bwd_status(sh, ws=None) == S.STILL_ERR_WORKSPACE
    # the routing to differentiate under is required once a chunk is complete
    assert bwd_status(sh, sel=None) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, sel=ct.c_void_p(0x1002)) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(shape(topk=0), sel=None, ws_bytes=16) == S.STILL_ERR_WORKSPACE
    assert bwd_status(shape(seqlen=40), sel=None, ws_bytes=16) == S.STILL_ERR_WORKSPACE  # N < C
    assert bwd_status(sh, ptr=None) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, ptr=MISALIGNED) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, dw=None) == S.STILL_ERR_INVALID_ARG
    # the forward's out and statistics come together, 16-byte aligned
    assert bwd_status(sh, out=FAKE) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, stats=FAKE) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, out=FAKE, stats=MISALIGNED) == S.STILL_ERR_INVALID_ARG
    # the forward's workspace must be as large as the forward needs (matrix-core
    # path; the fp32 kernels ignore it)
    fneed = S.fwd_workspace_size(sh)
    assert bwd_status(sh, fws=FAKE, fws_bytes=fneed - 1) == S.STILL_ERR_WORKSPACE
    for kw, st in ((dict(n_q_heads=6, n_kv_heads=4), S.STILL_ERR_INVALID_ARG),
                   (dict(head_dim=96), S.STILL_ERR_UNSUPPORTED)):
        assert bwd_status(shape(**kw)) == st
    timed = S.lib().still_hybrid_attn_bwd_timed
    n = ct.c_int32(0)
    evs = (ct.c_void_p * 4)()
    # up to 16 launches need one event more; too few is
    # rejected before anything runs
    assert timed(ct.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, None, 0,
                 FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None, evs, 4, ct.byref(n),
                 None) == S.STILL_ERR_INVALID_ARG


def test_bwd_empty_problem_without_projection_gradients_is_noop():
    for kw in (dict(seqlen=0), dict(batch=0)):
        assert bwd_status(shape(**kw), sel=None, ws=None, ws_bytes=0, ptr=None, dw=None) == S.STILL_OK


def test_future_utility_checks():
    sh = shape()
    n = ct.c_size_t(0)
    assert S.lib().still_future_kv_utility_workspace_size(ct.byref(sh), ct.byref(n)) == S.STILL_OK
    assert n.value >= 1 * 256 * 4 * 2 * 4
    f = S.lib().still_future_kv_utility
    assert f(ct.byref(sh), FAKE, FAKE, FAKE, FAKE, n.value - 1, None) == S.STILL_ERR_WORKSPACE
    assert f(ct.byref(sh), None, FAKE, FAKE, FAKE, n.value, None) == S.STILL_ERR_INVALID_ARG
    assert f(ct.byref(sh), MISALIGNED, FAKE, FAKE, FAKE, n.value, None) == S.STILL_ERR_INVALID_ARG
    assert f(ct.byref(sh), FAKE, FAKE, ct.c_void_p(0x1002), FAKE, n.value, None) == S.STILL_ERR_INVALID_ARG
    assert f(ct.byref(shape(head_dim=96)), FAKE, FAKE, FAKE, FAKE, n.value, None) == S.STILL_ERR_UNSUPPORTED
    assert f(ct.byref(shape(seqlen=0)), None, None, None, None, 0, None) == S.STILL_OK


def test_decode_rejects_misaligned_projections():
    sh = shape(seqlen=1, topk=32)
    need = 32 * ((16384 + 1 - 64 + 63) // 64)
    c = fake_cache(need, 16384)
    L = S.lib()
    for wq, wk in ((MISALIGNED, FAKE), (FAKE, MISALIGNED)):
        assert L.still_hybrid_attn_decode_step(ct.byref(sh), FAKE, FAKE, FAKE, wq, wk, None, ct.byref(c),
                                               FAKE, FAKE, 1 << 40, None) == S.STILL_ERR_INVALID_ARG


def test_noalloc_decode_checks_before_touching_the_gpu():
    """The no-allocation decode step validates like the plain step, and a
    step whose scratch need exceeds STILL_DECODE_SCRATCH_BYTES is refused
    with STILL_ERR_WORKSPACE before the scratch is looked up or anything is
    launched (no GPU here, so any HIP call would fail differently)."""
    L = S.lib()
    assert S.DECODE_SCRATCH_BYTES == 32 << 20
    sh = shape(batch=64, seqlen=1, n_q_heads=32, n_kv_heads=8)
    n = ct.c_size_t(0)
    # 64 sequences, 32 / 8 heads, d 128: a 8192-row cache fits, a 65536-row one does not
    for cap, fits in ((8192, True), (65536, False)):
        assert L.still_decode_workspace_size(ct.byref(sh), cap, ct.byref(n)) == S.STILL_OK
        assert (n.value <= S.DECODE_SCRATCH_BYTES) == fits
    cache = S.CacheStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 65536, FAKE, FAKE, 4096)
    st = L.still_hybrid_attn_decode_step_noalloc(ct.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                 ct.byref(cache), FAKE, None)
    assert st == S.STILL_ERR_WORKSPACE
    assert cache.pos == 4096
    # the plain step's argument checks come first
    assert L.still_hybrid_attn_decode_step_noalloc(ct.byref(sh), None, FAKE, FAKE, FAKE, FAKE, None,
                                                   ct.byref(cache), FAKE, None) == S.STILL_ERR_INVALID_ARG
    assert L.still_hybrid_attn_decode_step_noalloc(ct.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                   None, FAKE, None) == S.STILL_ERR_INVALID_ARG
    cache.pos = 1 << 40   # capacity: lambda * ceil((t + 1 - W) / C) > cap
    assert L.still_hybrid_attn_decode_step_noalloc(ct.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                   ct.byref(cache), FAKE, None) == S.STILL_ERR_CAPACITY


def test_gate_pointers_are_checked():
    """Gate logits (and their gradient) must be 4-byte aligned; NULL is no gate."""
    sh = shape()
    odd = ct.c_void_p(0x1002)
    assert fwd_status(sh, ws_bytes=16, gate=FAKE) == S.STILL_ERR_WORKSPACE   # accepted, then too small
    assert fwd_status(sh, gate=odd) == S.STILL_ERR_INVALID_ARG
    sd = shape(seqlen=1, topk=32)
    need = 32 * ((16384 + 1 - 64 + 63) // 64)
    assert decode_status(sd, fake_cache(need, 16384), gate=odd) == S.STILL_ERR_INVALID_ARG
    assert decode_status(sd, fake_cache(need, 16384), ws_bytes=16, gate=FAKE) == S.STILL_ERR_WORKSPACE
    assert bwd_status(sh, gate=odd) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, gate=FAKE, dgate=odd) == S.STILL_ERR_INVALID_ARG
    assert bwd_status(sh, gate=FAKE, dgate=FAKE, ws_bytes=16) == S.STILL_ERR_WORKSPACE
