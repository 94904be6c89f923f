"""Python binding of the STA C ABI (include/sta.h).

Argument marshalling only: shapes, dtypes and device pointers of torch
tensors are passed to libsta.so, which does every step of the computation
in its own HIP kernels.  PyTorch provides device memory and the stream.
"""

from __future__ import annotations

import contextlib
import ctypes
import math
from typing import Sequence

import torch

from . import _lib as L

__all__ = [
    "Plan", "sta_plan_create", "sta_tile_reorder", "sta_tile_unreorder", "sta_forward_plan",
    "sta_backward_plan", "sta_attention", "sta_forward", "sta_clear_plan_cache", "StaError",
    "window_candidates", "window_errors", "window_select", "window_search",
]

StaError = L.StaError

_DTYPES = {torch.bfloat16: L.STA_BF16, torch.float32: L.STA_F32}
_LAYOUTS = {"natural": L.STA_LAYOUT_NATURAL, "tile_major": L.STA_LAYOUT_TILE_MAJOR}


def _ints(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_int * len(xs))(*xs)


def _flat_windows(windows, heads: int):
    ws = [tuple(int(v) for v in w) for w in windows]
    if len(ws) == 1 and heads > 1:
        ws = ws * heads
    if len(ws) != heads or any(len(w) != 3 for w in ws):
        raise ValueError("windows: one (wT, wH, wW) per head")
    return [v for w in ws for v in w]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Buffers allocated for a call belong to the stream the call runs on:
    the caching allocator then hands a freed buffer (the backward's delta)
    only to later work on that stream, never to other streams while the
    call's kernels still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


@contextlib.contextmanager
def _scope(tensors, stream):
    """Every tensor of a call (and its stream, if given) must be on one
    device; the call allocates and launches with that device current."""
    dev = tensors[0].device
    for x in tensors[1:]:
        if x is not None and x.device != dev:
            raise ValueError(f"all tensors must be on {dev} (found {x.device})")
    if stream is not None and stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    with torch.cuda.device(dev), _on(stream):
        yield


class Plan:
    """Owned sta_plan handle (host tables; device tables are uploaded lazily)."""

    def __init__(self, batch: int, heads: int, video: Sequence[int], tile: Sequence[int],
                 windows, head_dim: int, partial_tiles: bool = False, token_windows: bool = False):
        """token_windows=True: a token-wise sliding-window (SWA) plan whose
        windows are in tokens; tile then only groups queries into work items."""
        h = ctypes.c_void_p()
        T, H, W = (int(x) for x in video)
        args = (int(batch), int(heads), T, H, W, _ints(tile), _ints(_flat_windows(windows, heads)),
                int(head_dim))
        if token_windows:
            st = L.lib().sta_swa_plan_create(*args, ctypes.byref(h))
        elif partial_tiles:
            st = L.lib().sta_plan_create_ex(*args, L.STA_PLAN_PARTIAL_TILES, ctypes.byref(h))
        else:
            st = L.lib().sta_plan_create(*args, ctypes.byref(h))
        L.check(st, "sta_plan_create")
        self._h = h
        self._destroy = L.lib().sta_plan_destroy
        self.info = L.PlanInfo()
        L.check(L.lib().sta_plan_get_info(self._h, ctypes.byref(self.info)), "sta_plan_get_info")

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._destroy(h)
            self._h = None

    # -- host queries -------------------------------------------------------
    @property
    def tokens(self) -> int:
        return int(self.info.tokens)

    @property
    def flops(self) -> float:
        return float(self.info.flops)

    def perm(self) -> torch.Tensor:
        out = torch.empty(self.tokens, dtype=torch.int32)
        L.check(L.lib().sta_plan_perm(self._h, ctypes.cast(out.data_ptr(), L._I32P), out.numel()),
                "sta_plan_perm")
        return out

    def kv_tiles(self, head: int, q_tile: int) -> list[int]:
        cnt = ctypes.c_int()
        L.lib().sta_plan_kv_tiles(self._h, head, q_tile, None, 0, ctypes.byref(cnt))
        buf = (ctypes.c_int32 * max(1, cnt.value))()
        L.check(L.lib().sta_plan_kv_tiles(self._h, head, q_tile, buf, cnt.value, ctypes.byref(cnt)),
                "sta_plan_kv_tiles")
        return list(buf[:cnt.value])

    def walk(self, which: int, head: int, tile: int) -> list[int]:
        """The lists in kernel walk order: which=0, the key tiles of query
        tile ``tile``; which=1, the query tiles that see key tile ``tile``."""
        cnt = ctypes.c_int()
        L.lib().sta_plan_walk(self._h, which, head, tile, None, 0, ctypes.byref(cnt))
        buf = (ctypes.c_int32 * max(1, cnt.value))()
        L.check(L.lib().sta_plan_walk(self._h, which, head, tile, buf, cnt.value, ctypes.byref(cnt)),
                "sta_plan_walk")
        return list(buf[:cnt.value])

    def q_tiles(self, head: int, kv_tile: int) -> list[int]:
        cnt = ctypes.c_int()
        L.lib().sta_plan_q_tiles(self._h, head, kv_tile, None, 0, ctypes.byref(cnt))
        buf = (ctypes.c_int32 * max(1, cnt.value))()
        L.check(L.lib().sta_plan_q_tiles(self._h, head, kv_tile, buf, cnt.value, ctypes.byref(cnt)),
                "sta_plan_q_tiles")
        return list(buf[:cnt.value])

    def schedule_bwd(self, which: int) -> torch.Tensor:
        """Backward launch schedule: which = 0 (dQ) or 1 (dK/dV)."""
        n = ctypes.c_int64()
        L.lib().sta_plan_schedule_bwd(self._h, which, None, 0, ctypes.byref(n))
        out = torch.empty(max(1, n.value), dtype=torch.int32)
        L.check(L.lib().sta_plan_schedule_bwd(self._h, which, ctypes.cast(out.data_ptr(), L._I32P),
                                              n.value, ctypes.byref(n)), "sta_plan_schedule_bwd")
        return out[:n.value]

    def schedule(self) -> torch.Tensor:
        n = ctypes.c_int64()
        L.lib().sta_plan_schedule(self._h, None, 0, ctypes.byref(n))
        out = torch.empty(n.value, dtype=torch.int32)
        L.check(L.lib().sta_plan_schedule(self._h, ctypes.cast(out.data_ptr(), L._I32P), n.value,
                                          ctypes.byref(n)), "sta_plan_schedule")
        return out

    def pieces(self) -> torch.Tensor:
        """[pieces, 5] int32: (item code, first step, end step, split item,
        pieces of that item) of every piece of a split work item."""
        n = ctypes.c_int64()
        L.lib().sta_plan_pieces(self._h, None, 0, ctypes.byref(n))
        out = torch.empty((max(1, n.value), 5), dtype=torch.int32)
        L.check(L.lib().sta_plan_pieces(self._h, ctypes.cast(out.data_ptr(), L._I32P), n.value,
                                        ctypes.byref(n)), "sta_plan_pieces")
        return out[:n.value]

    def group_lists(self) -> torch.Tensor:
        """Offsets of the per-work-group lists into schedule() (launch_blocks
        + 1 of them), or an empty tensor when the forward uses queues."""
        n = ctypes.c_int64()
        L.lib().sta_plan_group_lists(self._h, None, 0, ctypes.byref(n))
        out = torch.empty(max(1, n.value), dtype=torch.int32)
        L.check(L.lib().sta_plan_group_lists(self._h, ctypes.cast(out.data_ptr(), L._I32P), n.value,
                                             ctypes.byref(n)), "sta_plan_group_lists")
        return out[:n.value]


def sta_plan_create(batch, heads, video, tile, windows, head_dim) -> Plan:
    return Plan(batch, heads, video, tile, windows, head_dim)


def _check_tensor(x: torch.Tensor, plan: Plan, name: str):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.dtype not in _DTYPES:
        raise ValueError(f"{name}: dtype must be bfloat16 or float32")
    i = plan.info
    if x.numel() != i.batch * i.heads * i.tokens * i.head_dim:
        raise ValueError(f"{name}: expected {i.batch}x{i.heads}x{i.tokens}x{i.head_dim} elements")


def _reorder(fn, plan: Plan, x: torch.Tensor, out, stream):
    _check_tensor(x, plan, "x")
    with _scope([x, out], stream):
        if out is None:
            out = torch.empty_like(x)
        _check_tensor(out, plan, "out")
        if out.dtype != x.dtype:
            raise ValueError("out must have the input's dtype")
        L.check(fn(plan.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                   _DTYPES[x.dtype], _stream(stream)), fn.__name__)
    return out


def sta_tile_reorder(plan: Plan, x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Natural [B, heads, T, H, W, D] (or [B, heads, N, D]) -> tile-major [B, heads, N, D]."""
    y = _reorder(L.lib().sta_tile_reorder, plan, x, out, stream)
    return y.view(x.shape[0], x.shape[1], -1, x.shape[-1]) if out is None else y


def sta_tile_unreorder(plan: Plan, x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Tile-major [B, heads, N, D] -> natural order, same element count."""
    return _reorder(L.lib().sta_tile_unreorder, plan, x, out, stream)


def _check_rows(x: torch.Tensor, plan: Plan, name: str):
    i = plan.info
    if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous() \
            or x.dtype != torch.float32 or x.numel() != i.batch * i.heads * i.tokens:
        raise ValueError(f"{name}: contiguous CUDA float32 tensor of batch*heads*N elements required")


def _ptr(x):
    return ctypes.c_void_p(x.data_ptr())


def sta_forward_plan(plan: Plan, q, k, v, out=None, scale: float | None = None,
                     out_dtype=torch.float32, layout: str = "natural", stream=None, lse=None):
    """STA forward with a plan.  When ``lse`` is given ([B, heads, N]-sized
    float32 tensor, or True to allocate one) the row log-sum-exp is written
    too and ``(out, lse)`` is returned."""
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(x, plan, name)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(plan.info.head_dim)
    with _scope([q, k, v, out, lse if isinstance(lse, torch.Tensor) else None], stream):
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        _check_tensor(out, plan, "out")
        args = (plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out))
        tail = (float(scale), _DTYPES[q.dtype], _DTYPES[out.dtype], _LAYOUTS[layout], _stream(stream))
        if lse is None or lse is False:
            L.check(L.lib().sta_forward_plan(*args, *tail), "sta_forward_plan")
            return out
        if lse is True:
            i = plan.info
            lse = torch.empty((i.batch, i.heads, i.tokens), dtype=torch.float32, device=q.device)
        _check_rows(lse, plan, "lse")
        L.check(L.lib().sta_forward_plan_lse(*args, _ptr(lse), *tail), "sta_forward_plan_lse")
    return out, lse


def sta_backward_plan(plan: Plan, q, k, v, out, dout, lse, scale: float | None = None,
                      grad_dtype=torch.float32, layout: str = "natural", dq=None, dk=None, dv=None,
                      delta=None, stream=None):
    """STA backward: (dq, dk, dv) of <out, dout>.  ``out`` and ``lse`` come
    from ``sta_forward_plan(..., lse=True)`` on the same inputs."""
    for name, x in (("q", q), ("k", k), ("v", v), ("dout", dout), ("out", out)):
        _check_tensor(x, plan, name)
    if not (q.dtype == k.dtype == v.dtype == dout.dtype):
        raise ValueError("q, k, v, dout must share a dtype")
    _check_rows(lse, plan, "lse")
    i = plan.info
    if scale is None:
        scale = 1.0 / math.sqrt(i.head_dim)
    with _scope([q, k, v, out, dout, lse, delta, dq, dk, dv], stream):
        if delta is None:
            delta = torch.empty((i.batch, i.heads, i.tokens), dtype=torch.float32, device=q.device)
        _check_rows(delta, plan, "delta")
        grads = []
        for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
            if g is None:
                g = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
            _check_tensor(g, plan, name)
            grads.append(g)
        if not (grads[0].dtype == grads[1].dtype == grads[2].dtype):
            raise ValueError("dq, dk, dv must share a dtype")
        st = L.lib().sta_backward_plan(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                       _ptr(lse), _ptr(delta), *(_ptr(g) for g in grads), float(scale),
                                       _DTYPES[q.dtype], _DTYPES[out.dtype], _DTYPES[grads[0].dtype],
                                       _LAYOUTS[layout], _stream(stream))
        L.check(st, "sta_backward_plan")
    return tuple(grads)


class _StaAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, plan, scale, layout):
        q, k, v = (x.contiguous() for x in (q, k, v))
        out, lse = sta_forward_plan(plan, q, k, v, scale=scale, out_dtype=q.dtype, layout=layout,
                                    lse=True)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.plan, ctx.scale, ctx.layout = plan, scale, layout
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv = sta_backward_plan(ctx.plan, q, k, v, out, dout.contiguous().to(q.dtype), lse,
                                       scale=ctx.scale, grad_dtype=q.dtype, layout=ctx.layout)
        return dq, dk, dv, None, None, None


def sta_attention(q, k, v, plan: Plan, scale: float | None = None, layout: str = "natural"):
    """Differentiable STA (autograd through the library's forward and
    backward).  Output and gradients have q's dtype."""
    if scale is None:
        scale = 1.0 / math.sqrt(plan.info.head_dim)
    return _StaAttention.apply(q, k, v, plan, float(scale), layout)


def _video_inputs(q, k, v, video):
    """(B, heads, T, H, W, D) of natural-order q, k, v given as
    [B, heads, T, H, W, D], or as [B, heads, N, D] with video=(T, H, W)."""
    if not isinstance(q, torch.Tensor) or q.dim() not in (4, 6):
        raise ValueError("q must be a [B, heads, T, H, W, D] or [B, heads, N, D] tensor")
    if q.dim() == 6:
        B, heads, T, H, W, D = q.shape
    else:
        if video is None:
            raise ValueError("video=(T, H, W) is required for 4-D inputs")
        B, heads, N, D = q.shape
        T, H, W = (int(x) for x in video)
        if N != T * H * W:
            raise ValueError(f"q has {N} tokens, video {T}x{H}x{W} has {T * H * W}")
    for name, x in (("q", q), ("k", k), ("v", v)):
        if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous() \
                or x.dtype not in _DTYPES or x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{name}: contiguous CUDA bf16/fp32 tensor shaped like q (and of its dtype) required")
    return B, heads, T, H, W, D


def sta_forward(q, k, v, tile, windows, scale: float | None = None, out=None,
                out_dtype=torch.float32, layout: str = "natural", video=None, stream=None):
    """STA forward through the library's plan cache.

    q, k, v: [B, heads, T, H, W, D] (natural layout), or [B, heads, N, D]
    with ``video=(T, H, W)``.  windows: one (wT, wH, wW) per head (or one for
    all heads), in tiles."""
    B, heads, T, H, W, D = _video_inputs(q, k, v, video)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with _scope([q, k, v, out], stream):
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        if not out.is_cuda or not out.is_contiguous() or out.dtype not in _DTYPES or out.numel() != q.numel():
            raise ValueError("out: contiguous CUDA bf16/fp32 tensor with q's element count required")
        st = L.lib().sta_forward(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                 ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                 int(B), int(heads), int(T), int(H), int(W), _ints(tile),
                                 _ints(_flat_windows(windows, heads)), int(D), float(scale),
                                 _DTYPES[q.dtype], _DTYPES[out.dtype], _LAYOUTS[layout], _stream(stream))
        L.check(st, "sta_forward")
    return out


def window_candidates(grid) -> list[tuple[int, int, int]]:
    """The library's default candidate windows for a tile grid."""
    g = _ints(grid)
    cnt = ctypes.c_int()
    L.lib().sta_window_candidates(g, None, 0, ctypes.byref(cnt))
    buf = (ctypes.c_int * (3 * max(1, cnt.value)))()
    L.check(L.lib().sta_window_candidates(g, buf, cnt.value, ctypes.byref(cnt)), "sta_window_candidates")
    return [tuple(buf[3 * i:3 * i + 3]) for i in range(cnt.value)]


def window_errors(q, k, v, tile, candidates, scale: float | None = None, layout: str = "natural",
                  video=None, stream=None):
    """[heads, n_cand] relative errors of STA against full attention for
    each candidate window, on one calibration input (natural
    [B, heads, T, H, W, D], or [B, heads, N, D] with video=(T, H, W))."""
    import numpy as np
    B, heads, T, H, W, D = _video_inputs(q, k, v, video)
    cands = [tuple(int(x) for x in w) for w in candidates]
    if not cands or any(len(w) != 3 for w in cands):
        raise ValueError("candidates: one or more (wT, wH, wW) windows")
    n = len(cands)
    err = (ctypes.c_double * (heads * n))()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with _scope([q, k, v], stream):
        st = L.lib().sta_window_errors(_ptr(q), _ptr(k), _ptr(v), int(B), int(heads), int(T), int(H), int(W),
                                       _ints(tile), int(D), float(scale), _DTYPES[q.dtype], _LAYOUTS[layout],
                                       _ints([x for w in cands for x in w]), n, err, _stream(stream))
        L.check(st, "sta_window_errors")
    return np.array(err[:], dtype=np.float64).reshape(heads, n)


def window_select(err, candidates, grid, threshold: float) -> list[tuple[int, int, int]]:
    """Per head, the cheapest candidate within threshold (else the grid)."""
    import numpy as np
    err = np.ascontiguousarray(err, dtype=np.float64)
    heads, n = err.shape
    cands = [int(x) for w in candidates for x in w]
    if len(cands) != 3 * n:
        raise ValueError("one error column per candidate")
    out = (ctypes.c_int * (3 * heads))()
    st = L.lib().sta_window_select(heads, _ints(grid), _ints(cands), n,
                                   err.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), float(threshold),
                                   out)
    L.check(st, "sta_window_select")
    return [tuple(out[3 * h:3 * h + 3]) for h in range(heads)]


def window_search(samples, tile, threshold: float, candidates=None, scale: float | None = None,
                  layout: str = "natural", stream=None):
    """Per-head windows from calibration inputs (``sta_window_search``):
    ``samples`` is a sequence of (q, k, v) in natural [B, heads, T, H, W, D]
    order, all of one shape and dtype.  The library averages the errors over
    the samples before the choice.  Returns (windows, mean errors,
    candidates)."""
    import numpy as np
    samples = [tuple(s) for s in samples]
    if not samples:
        raise ValueError("no calibration samples")
    shapes = {tuple(x.shape) for s in samples for x in s}
    dtypes = {x.dtype for s in samples for x in s}
    if len(shapes) != 1 or len(dtypes) != 1:
        raise ValueError("calibration samples must share one shape and dtype")
    for s in samples:
        _video_inputs(*s, None)
    q0, k0, v0 = samples[0]
    B, heads, T, H, W, D = _video_inputs(q0, k0, v0, None)
    grid = tuple(-(-e // t) for e, t in zip((T, H, W), tile))   # partial tiles at the far edges count
    cands = [tuple(int(x) for x in w) for w in (candidates if candidates is not None else window_candidates(grid))]
    n = len(cands)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    arr = [(ctypes.c_void_p * len(samples))(*(_ptr(s[i]) for s in samples)) for i in range(3)]
    err = (ctypes.c_double * (heads * n))()
    out = (ctypes.c_int * (3 * heads))()
    with _scope([x for s in samples for x in s], stream):
        st = L.lib().sta_window_search(*arr, len(samples), int(B), int(heads), int(T), int(H), int(W),
                                       _ints(tile), int(D), float(scale), _DTYPES[q0.dtype], _LAYOUTS[layout],
                                       _ints([x for w in cands for x in w]), n, float(threshold), err, out,
                                       _stream(stream))
        L.check(st, "sta_window_search")
    windows = [tuple(out[3 * h:3 * h + 3]) for h in range(heads)]
    return windows, np.array(err[:], dtype=np.float64).reshape(heads, n), cands


def sta_clear_plan_cache() -> None:
    L.check(L.lib().sta_clear_plan_cache(), "sta_clear_plan_cache")
