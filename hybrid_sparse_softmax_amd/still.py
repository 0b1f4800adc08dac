"""Python binding of libstill: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI declared in
include/still.h; PyTorch supplies device memory and the current stream.  The
names follow the C entry points.  There is no fallback: if the library is
not built, every call raises.
"""
from __future__ import annotations

import ctypes as ct
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libstill.so")

STILL_OK, STILL_ERR_INVALID_ARG, STILL_ERR_UNSUPPORTED = 0, -1, -2
STILL_ERR_WORKSPACE, STILL_ERR_CAPACITY, STILL_ERR_HIP = -3, -4, -5
STILL_F32, STILL_BF16 = 0, 1
STILL_FLAG_GENERAL_KERNELS = 1
STILL_ROUTE_SHIFT = 1
# routing criteria (STILL_ROUTE_* of still.h), by name
ROUTES = {"saliency": 0, "diagonal": 1, "qk": 2, "keynorm": 3, "uniform": 4, "random": 5}

STILL_MAX_LAUNCHES = 24

EXPORTED = (
    "still_abi_version", "still_status_str", "still_topk_for_budget",
    "still_fwd_workspace_size", "still_hybrid_attn_fwd",
    "still_decode_workspace_size", "still_hybrid_attn_decode_step",
    "still_hybrid_attn_fwd_timed", "still_hybrid_attn_decode_step_timed",
    "still_hybrid_attn_decode_step_ragged", "still_hybrid_attn_decode_step_noalloc",
    "still_bwd_workspace_size", "still_hybrid_attn_bwd", "still_hybrid_attn_bwd_timed",
    "still_future_kv_utility_workspace_size", "still_future_kv_utility",
)


class StillError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


class Shape(ct.Structure):
    _fields_ = [("batch", ct.c_int32), ("seqlen", ct.c_int32), ("n_q_heads", ct.c_int32),
                ("n_kv_heads", ct.c_int32), ("head_dim", ct.c_int32), ("feat_dim", ct.c_int32),
                ("window", ct.c_int32), ("chunk", ct.c_int32), ("topk", ct.c_int32),
                ("eps", ct.c_float), ("softmax_scale", ct.c_float), ("dtype", ct.c_int32),
                ("flags", ct.c_uint32)]


class CacheStruct(ct.Structure):
    _fields_ = [("win_k", ct.c_void_p), ("win_v", ct.c_void_p), ("win_route", ct.c_void_p),
                ("pend_score", ct.c_void_p), ("sel_k", ct.c_void_p), ("sel_v", ct.c_void_p),
                ("sel_count", ct.c_void_p), ("sel_cap", ct.c_int32), ("lin_S", ct.c_void_p),
                ("lin_z", ct.c_void_p), ("pos", ct.c_int64)]


_lib = None


def lib() -> ct.CDLL:
    """Load libstill.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hybrid_sparse_softmax_amd.build`")
        L = ct.CDLL(LIB_PATH)
        vp, sz = ct.c_void_p, ct.c_size_t
        L.still_abi_version.restype = ct.c_int32
        L.still_abi_version.argtypes = []
        L.still_status_str.restype = ct.c_char_p
        L.still_status_str.argtypes = [ct.c_int]
        L.still_topk_for_budget.restype = ct.c_int32
        L.still_topk_for_budget.argtypes = [ct.c_int32, ct.c_int32, ct.c_int32, ct.c_int64]
        L.still_fwd_workspace_size.restype = ct.c_int
        L.still_fwd_workspace_size.argtypes = [ct.POINTER(Shape), ct.POINTER(sz)]
        L.still_hybrid_attn_fwd.restype = ct.c_int
        L.still_hybrid_attn_fwd.argtypes = [ct.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, ct.POINTER(CacheStruct), vp, sz, vp]
        L.still_decode_workspace_size.restype = ct.c_int
        L.still_decode_workspace_size.argtypes = [ct.POINTER(Shape), ct.c_int32, ct.POINTER(sz)]
        L.still_hybrid_attn_decode_step.restype = ct.c_int
        L.still_hybrid_attn_decode_step.argtypes = [ct.POINTER(Shape), vp, vp, vp, vp, vp, vp,
                                                    ct.POINTER(CacheStruct), vp, vp, sz, vp]
        L.still_hybrid_attn_decode_step_noalloc.restype = ct.c_int
        L.still_hybrid_attn_decode_step_noalloc.argtypes = [ct.POINTER(Shape), vp, vp, vp, vp, vp,
                                                            vp, ct.POINTER(CacheStruct), vp, vp]
        L.still_hybrid_attn_decode_step_ragged.restype = ct.c_int
        L.still_hybrid_attn_decode_step_ragged.argtypes = [ct.POINTER(Shape), vp, vp, vp, vp, vp,
                                                           vp, ct.POINTER(CacheStruct), vp,
                                                           ct.c_int64, vp, vp, sz, vp]
        L.still_bwd_workspace_size.restype = ct.c_int
        L.still_bwd_workspace_size.argtypes = [ct.POINTER(Shape), ct.POINTER(sz)]
        L.still_hybrid_attn_bwd.restype = ct.c_int
        L.still_hybrid_attn_bwd.argtypes = [ct.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, vp, sz, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.still_future_kv_utility_workspace_size.restype = ct.c_int
        L.still_future_kv_utility_workspace_size.argtypes = [ct.POINTER(Shape), ct.POINTER(sz)]
        L.still_future_kv_utility.restype = ct.c_int
        L.still_future_kv_utility.argtypes = [ct.POINTER(Shape), vp, vp, vp, vp, sz, vp]
        ev = [ct.POINTER(ct.c_void_p), ct.c_int32, ct.POINTER(ct.c_int32), ct.POINTER(ct.c_char_p)]
        L.still_hybrid_attn_bwd_timed.restype = ct.c_int
        L.still_hybrid_attn_bwd_timed.argtypes = L.still_hybrid_attn_bwd.argtypes + ev
        L.still_hybrid_attn_fwd_timed.restype = ct.c_int
        L.still_hybrid_attn_fwd_timed.argtypes = L.still_hybrid_attn_fwd.argtypes + ev
        L.still_hybrid_attn_decode_step_timed.restype = ct.c_int
        L.still_hybrid_attn_decode_step_timed.argtypes = L.still_hybrid_attn_decode_step.argtypes + ev
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().still_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib().still_abi_version())


def topk_for_budget(m: int, window: int, chunk: int, n_max: int) -> int:
    return int(lib().still_topk_for_budget(m, window, chunk, n_max))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return STILL_BF16
    if dt == torch.float32:
        return STILL_F32
    raise TypeError(f"unsupported dtype {dt}")


def make_shape(*, batch, seqlen, n_q_heads, n_kv_heads, head_dim, window, chunk, topk,
               eps=1e-6, softmax_scale=0.0, dtype=torch.bfloat16, feat_dim=None,
               general=False, route="saliency") -> Shape:
    flags = (STILL_FLAG_GENERAL_KERNELS if general else 0) | (ROUTES[route] << STILL_ROUTE_SHIFT)
    return Shape(batch, seqlen, n_q_heads, n_kv_heads, head_dim,
                 head_dim if feat_dim is None else feat_dim, window, chunk, topk, eps,
                 softmax_scale, _dtype_code(dtype), flags)


def _ptr(t):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream():
    return ct.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != STILL_OK:
        raise StillError(status, where)


def fwd_workspace_size(shape: Shape) -> int:
    n = ct.c_size_t(0)
    _check(lib().still_fwd_workspace_size(ct.byref(shape), ct.byref(n)), "still_fwd_workspace_size")
    return n.value


def bwd_workspace_size(shape: Shape) -> int:
    n = ct.c_size_t(0)
    _check(lib().still_bwd_workspace_size(ct.byref(shape), ct.byref(n)), "still_bwd_workspace_size")
    return n.value


def decode_workspace_size(shape: Shape, sel_cap: int) -> int:
    n = ct.c_size_t(0)
    _check(lib().still_decode_workspace_size(ct.byref(shape), sel_cap, ct.byref(n)),
           "still_decode_workspace_size")
    return n.value


def _expect(t, name, dtype, shape):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: want contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


class LaunchTimer:
    """HIP events handed to the *_timed entry points: event i is recorded on
    the launch stream before kernel launch i, the last one after the final
    launch.  Events come from torch (each recorded once so it exists)."""

    def __init__(self, n_events: int = STILL_MAX_LAUNCHES + 1):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
        for e in self.events:
            e.record()
        torch.cuda.synchronize()
        self.handles = (ct.c_void_p * n_events)(*[e.cuda_event for e in self.events])
        self.names = (ct.c_char_p * n_events)()
        self.n = ct.c_int32(0)

    def args(self):
        return [self.handles, len(self.events), ct.byref(self.n), self.names]

    def durations_ms(self) -> list:
        """[(kernel name, milliseconds)] of the last timed call (synchronises)."""
        self.events[self.n.value].synchronize()
        return [(self.names[i].decode(), self.events[i].elapsed_time(self.events[i + 1]))
                for i in range(self.n.value)]


class DecodeCache:
    """Caller-owned decode cache tensors (layouts of still_cache)."""

    def __init__(self, *, batch, n_kv_heads, head_dim, window, chunk, topk, sel_cap,
                 dtype=torch.bfloat16, feat_dim=None, device="cuda", pos=0):
        fd = head_dim if feat_dim is None else feat_dim
        B, H, d, W, C = batch, n_kv_heads, head_dim, window, chunk
        self.window, self.chunk, self.topk = W, C, topk
        self.win_k = torch.zeros((B, H, max(W, 1), d), dtype=dtype, device=device)
        self.win_v = torch.zeros_like(self.win_k)
        self.win_route = torch.zeros((B, H, max(W, 1)), dtype=torch.uint8, device=device)
        self.pend_score = torch.zeros((B, H, C), dtype=torch.float32, device=device)
        self.sel_k = torch.zeros((B, H, max(sel_cap, 1), d), dtype=dtype, device=device)
        self.sel_v = torch.zeros_like(self.sel_k)
        self.sel_count = torch.zeros((B, H), dtype=torch.int32, device=device)
        self.sel_cap = sel_cap
        self.lin_S = torch.zeros((B, H, fd, d), dtype=torch.float32, device=device)
        self.lin_z = torch.zeros((B, H, fd), dtype=torch.float32, device=device)
        self.pos = pos
        self._struct = None

    def struct(self) -> CacheStruct:
        self._struct = CacheStruct(self.win_k.data_ptr(), self.win_v.data_ptr(),
                                   self.win_route.data_ptr(), self.pend_score.data_ptr(),
                                   self.sel_k.data_ptr(), self.sel_v.data_ptr(),
                                   self.sel_count.data_ptr(), self.sel_cap,
                                   self.lin_S.data_ptr(), self.lin_z.data_ptr(), self.pos)
        return self._struct

    def tensors(self) -> dict:
        return {k: getattr(self, k) for k in ("win_k", "win_v", "win_route", "pend_score", "sel_k",
                                              "sel_v", "sel_count", "lin_S", "lin_z")}


def fwd(q, k, v, wphi_q, wphi_k, *, window, chunk, topk, eps=1e-6, softmax_scale=0.0,
        return_scores=False, return_sel=False, return_stats=False, cache: DecodeCache | None = None,
        out=None, workspace=None, general=False, timer: LaunchTimer | None = None,
        route="saliency", gate=None, stats=None, return_workspace=False) -> dict:
    """still_hybrid_attn_fwd.  q [B,N,Hq,d], k/v [B,N,Hkv,d] (bf16 or f32),
    wphi_* [Hkv, d'/2, d] f32, gate: optional gate logits [B,N,Hq] f32.
    return_stats (or a given stats tensor [B,N,Hq,4] f32): the per-query
    statistics bwd can start from; return_workspace: the workspace tensor
    used, whose linear state bwd can reuse (fwd_workspace).  Returns
    dict(out, scores?, sel_idx?, stats?, workspace?)."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    sh = make_shape(batch=B, seqlen=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=window,
                    chunk=chunk, topk=topk, eps=eps, softmax_scale=softmax_scale, dtype=q.dtype,
                    feat_dim=2 * wphi_q.shape[1], general=general, route=route)
    _expect(q, "q", q.dtype, (B, N, Hq, d))
    _expect(k, "k", q.dtype, (B, N, Hkv, d))
    _expect(v, "v", q.dtype, (B, N, Hkv, d))
    _expect(wphi_q, "wphi_q", torch.float32, (Hkv, wphi_q.shape[1], d))
    _expect(wphi_k, "wphi_k", torch.float32, (Hkv, wphi_q.shape[1], d))
    if gate is not None:
        _expect(gate, "gate", torch.float32, (B, N, Hq))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lam = min(topk, chunk)
    scores = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev) if return_scores else None
    sel = torch.empty((B, Hkv, N // chunk, lam), dtype=torch.int32, device=dev) if return_sel else None
    if stats is not None:
        _expect(stats, "stats", torch.float32, (B, N, Hq, 4))
    elif return_stats:
        stats = torch.empty((B, N, Hq, 4), dtype=torch.float32, device=dev)
    nbytes = fwd_workspace_size(sh)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    cs = ct.byref(cache.struct()) if cache is not None else None
    args = [ct.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(wphi_q), _ptr(wphi_k), _ptr(gate),
            _ptr(out), _ptr(scores), _ptr(sel), _ptr(stats), cs, _ptr(workspace), workspace.numel(),
            _stream()]
    if timer is None:
        _check(lib().still_hybrid_attn_fwd(*args), "still_hybrid_attn_fwd")
    else:
        _check(lib().still_hybrid_attn_fwd_timed(*args, *timer.args()), "still_hybrid_attn_fwd_timed")
    res = {"out": out}
    if scores is not None:
        res["scores"] = scores
    if sel is not None:
        res["sel_idx"] = sel
    if stats is not None:
        res["stats"] = stats
    if return_workspace:
        res["workspace"] = workspace
    return res


def decode_step(q, k, v, wphi_q, wphi_k, cache: DecodeCache, *, eps=1e-6, softmax_scale=0.0,
                out=None, workspace=None, general=False, timer: LaunchTimer | None = None,
                route="saliency", gate=None):
    """still_hybrid_attn_decode_step at position cache.pos; q [B,1,Hq,d],
    k/v [B,1,Hkv,d], gate: optional gate logits [B,1,Hq] f32.  Advances
    cache.pos.  Returns out [B,1,Hq,d]."""
    B, one, Hq, d = q.shape
    Hkv = k.shape[2]
    sh = make_shape(batch=B, seqlen=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                    window=cache.window, chunk=cache.chunk, topk=cache.topk, eps=eps,
                    softmax_scale=softmax_scale, dtype=q.dtype, feat_dim=2 * wphi_q.shape[1],
                    general=general, route=route)
    _expect(q, "q", q.dtype, (B, 1, Hq, d))
    _expect(k, "k", q.dtype, (B, 1, Hkv, d))
    _expect(v, "v", q.dtype, (B, 1, Hkv, d))
    if out is None:
        out = torch.empty_like(q)
    nbytes = decode_workspace_size(sh, cache.sel_cap)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _gate_check(gate, B, Hq)
    args = [ct.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(wphi_q), _ptr(wphi_k), _ptr(gate),
            ct.byref(cs), _ptr(out), _ptr(workspace), workspace.numel(), _stream()]
    if timer is None:
        _check(lib().still_hybrid_attn_decode_step(*args), "still_hybrid_attn_decode_step")
    else:
        _check(lib().still_hybrid_attn_decode_step_timed(*args, *timer.args()),
               "still_hybrid_attn_decode_step_timed")
    cache.pos = int(cs.pos)
    return out


DECODE_SCRATCH_BYTES = 32 << 20  # STILL_DECODE_SCRATCH_BYTES


def _gate_check(gate, B, Hq):
    if gate is not None:
        _expect(gate, "gate", torch.float32, (B, 1, Hq))


def decode_step_noalloc(q, k, v, wphi_q, wphi_k, cache: DecodeCache, *, eps=1e-6,
                        softmax_scale=0.0, out=None, general=False, route="saliency", gate=None):
    """still_hybrid_attn_decode_step_noalloc: the decode step at cache.pos
    with the library's own per-GPU scratch instead of a workspace (nothing is
    allocated when ``out`` is given).  Advances cache.pos.  Returns out
    [B,1,Hq,d]."""
    B, one, Hq, d = q.shape
    Hkv = k.shape[2]
    sh = make_shape(batch=B, seqlen=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                    window=cache.window, chunk=cache.chunk, topk=cache.topk, eps=eps,
                    softmax_scale=softmax_scale, dtype=q.dtype, feat_dim=2 * wphi_q.shape[1],
                    general=general, route=route)
    _expect(q, "q", q.dtype, (B, 1, Hq, d))
    _expect(k, "k", q.dtype, (B, 1, Hkv, d))
    _expect(v, "v", q.dtype, (B, 1, Hkv, d))
    if out is None:
        out = torch.empty_like(q)
    _gate_check(gate, B, Hq)
    cs = cache.struct()
    _check(lib().still_hybrid_attn_decode_step_noalloc(
        ct.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(wphi_q), _ptr(wphi_k), _ptr(gate), ct.byref(cs),
        _ptr(out), _stream()), "still_hybrid_attn_decode_step_noalloc")
    cache.pos = int(cs.pos)
    return out


def decode_step_ragged(q, k, v, wphi_q, wphi_k, cache: DecodeCache, pos: torch.Tensor, max_pos: int,
                       *, eps=1e-6, softmax_scale=0.0, out=None, workspace=None, general=False,
                       route="saliency", gate=None):
    """still_hybrid_attn_decode_step_ragged: one step with a position per
    sequence.  pos is an int64 device tensor [B] (advanced by one on the
    stream), max_pos a host bound on its entries; cache.pos is not used.
    q [B,1,Hq,d], k/v [B,1,Hkv,d].  Returns out [B,1,Hq,d]."""
    B, one, Hq, d = q.shape
    Hkv = k.shape[2]
    sh = make_shape(batch=B, seqlen=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                    window=cache.window, chunk=cache.chunk, topk=cache.topk, eps=eps,
                    softmax_scale=softmax_scale, dtype=q.dtype, feat_dim=2 * wphi_q.shape[1],
                    general=general, route=route)
    _expect(q, "q", q.dtype, (B, 1, Hq, d))
    _expect(k, "k", q.dtype, (B, 1, Hkv, d))
    _expect(v, "v", q.dtype, (B, 1, Hkv, d))
    _expect(pos, "pos", torch.int64, (B,))
    if out is None:
        out = torch.empty_like(q)
    nbytes = decode_workspace_size(sh, cache.sel_cap)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _gate_check(gate, B, Hq)
    cs = cache.struct()
    _check(lib().still_hybrid_attn_decode_step_ragged(
        ct.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(wphi_q), _ptr(wphi_k), _ptr(gate), ct.byref(cs),
        _ptr(pos),
        int(max_pos), _ptr(out), _ptr(workspace), workspace.numel(), _stream()),
        "still_hybrid_attn_decode_step_ragged")
    return out


def bwd(q, k, v, wphi_q, wphi_k, sel_idx, dout, *, window, chunk, topk, eps=1e-6,
        softmax_scale=0.0, workspace=None, timer: LaunchTimer | None = None, gate=None,
        general=False, out=None, stats=None, fwd_workspace=None) -> dict:
    """still_hybrid_attn_bwd: gradients of sum(dout * out) for the forward
    with the same arguments, under the routing sel_idx [B, Hkv, N/C, lambda]
    (the forward's sel_idx output; None when there is nothing selected).
    out, stats: the forward's output and return_stats tensor, both or
    neither.  fwd_workspace: the workspace tensor of that forward call
    (untouched since), whose linear state the backward then reuses.  Returns dict(dq, dk, dv, dwphi_q, dwphi_k), all fp32, plus
    dgate [B, N, Hq] when gate logits [B, N, Hq] are given."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    sh = make_shape(batch=B, seqlen=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=window,
                    chunk=chunk, topk=topk, eps=eps, softmax_scale=softmax_scale, dtype=q.dtype,
                    feat_dim=2 * wphi_q.shape[1], general=general)
    _expect(q, "q", q.dtype, (B, N, Hq, d))
    _expect(k, "k", q.dtype, (B, N, Hkv, d))
    _expect(v, "v", q.dtype, (B, N, Hkv, d))
    _expect(dout, "dout", q.dtype, (B, N, Hq, d))
    _expect(wphi_q, "wphi_q", torch.float32, (Hkv, wphi_q.shape[1], d))
    _expect(wphi_k, "wphi_k", torch.float32, (Hkv, wphi_q.shape[1], d))
    if sel_idx is not None:
        _expect(sel_idx, "sel_idx", torch.int32, (B, Hkv, N // chunk, min(topk, chunk)))
    if out is not None:
        _expect(out, "out", q.dtype, (B, N, Hq, d))
    if stats is not None:
        _expect(stats, "stats", torch.float32, (B, N, Hq, 4))
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(k.shape, **f32),
           "dv": torch.empty(v.shape, **f32), "dwphi_q": torch.empty(wphi_q.shape, **f32),
           "dwphi_k": torch.empty(wphi_k.shape, **f32)}
    if gate is not None:
        _expect(gate, "gate", torch.float32, (B, N, Hq))
        res["dgate"] = torch.empty(gate.shape, **f32)
    nbytes = bwd_workspace_size(sh)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = [ct.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(wphi_q), _ptr(wphi_k), _ptr(gate),
            _ptr(sel_idx), _ptr(dout), _ptr(out), _ptr(stats), _ptr(fwd_workspace),
            0 if fwd_workspace is None else fwd_workspace.numel(), _ptr(res["dq"]), _ptr(res["dk"]),
            _ptr(res["dv"]),
            _ptr(res["dwphi_q"]), _ptr(res["dwphi_k"]), _ptr(res.get("dgate")), _ptr(workspace),
            workspace.numel(), _stream()]
    if timer is None:
        _check(lib().still_hybrid_attn_bwd(*args), "still_hybrid_attn_bwd")
    else:
        _check(lib().still_hybrid_attn_bwd_timed(*args, *timer.args()), "still_hybrid_attn_bwd_timed")
    return res


def future_kv_utility(q, k, *, window, chunk=64, softmax_scale=0.0, workspace=None):
    """still_future_kv_utility: util [B, Hkv, N] fp32, the full causal
    attention weight each key receives from the queries after its window,
    summed over the group's query heads."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    sh = make_shape(batch=B, seqlen=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=window,
                    chunk=chunk, topk=0, softmax_scale=softmax_scale, dtype=q.dtype)
    _expect(q, "q", q.dtype, (B, N, Hq, d))
    _expect(k, "k", q.dtype, (B, N, Hkv, d))
    util = torch.empty((B, Hkv, N), dtype=torch.float32, device=q.device)
    n = ct.c_size_t(0)
    _check(lib().still_future_kv_utility_workspace_size(ct.byref(sh), ct.byref(n)),
           "still_future_kv_utility_workspace_size")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
    _check(lib().still_future_kv_utility(ct.byref(sh), _ptr(q), _ptr(k), _ptr(util), _ptr(workspace),
                                         workspace.numel(), _stream()), "still_future_kv_utility")
    return util
