"""ctypes binding of libhga.so: the C ABI in include/hga.h, same names.

Argument marshalling only: torch tensors are passed as device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhga.so")

HGA_F32 = 0
HGA_BF16 = 1
HGA_MAX_CHUNKS = 8192

STATUS = {
    0: "HGA_OK", -1: "HGA_ERR_NULL", -2: "HGA_ERR_SHAPE", -3: "HGA_ERR_UNSUPPORTED",
    -4: "HGA_ERR_CAPACITY", -5: "HGA_ERR_ALIGN", -6: "HGA_ERR_WORKSPACE", -7: "HGA_ERR_HIP",
}


class HgaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


class HgaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("chunk", ctypes.c_int32), ("group", ctypes.c_int32),
        ("q_block", ctypes.c_int32), ("top_chunks", ctypes.c_int32), ("top_groups", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
    ]


_DTYPE_CODES = {"bf16": HGA_BF16, "f32": HGA_F32}


def make_shape(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, top_chunks: int,
               top_groups: int, dtype: str = "bf16", softmax_scale: float = 0.0) -> HgaShape:
    """The hga_shape of a call; dtype is "bf16" or "f32" (anything else raises)."""
    if dtype not in _DTYPE_CODES:
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    return HgaShape(batch, n_q_heads, n_kv_heads, head_dim, 64, 8, 64, top_chunks, top_groups,
                    _DTYPE_CODES[dtype], softmax_scale)


def _float_dtype(shape: HgaShape) -> torch.dtype:
    return torch.bfloat16 if shape.dtype == HGA_BF16 else torch.float32


def _need(fn: str, name: str, t: Optional[torch.Tensor], dtype: torch.dtype, numel: int, device,
          optional: bool = False) -> None:
    """Host-side check of one tensor argument before its pointer crosses the C ABI:
    the library trusts pointers, so a tensor of the wrong dtype, layout, device or
    size would become an out-of-bounds device access instead of an error."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{fn}: {name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{fn}: {name} is on {t.device}, expected {device}")
    if t.numel() != numel:
        raise ValueError(f"{fn}: {name} has {t.numel()} elements, expected {numel}")


def _dev_of(*ts) -> torch.device:
    for t in ts:
        if isinstance(t, torch.Tensor):
            if t.device.type != "cuda":
                raise ValueError(f"tensors must be on a ROCm device, got {t.device}")
            return t.device
    raise ValueError("no tensor arguments")


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SHAPE = ctypes.POINTER(HgaShape)

SIGNATURES = {
    "hga_build_summaries": (ctypes.c_int, [_SHAPE, _P, _I64, _I64, _I64, _P, _P, _P]),
    "hga_route": (ctypes.c_int, [_SHAPE, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "hga_route_causal": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "hga_attend_fwd": (ctypes.c_int, [_SHAPE, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "hga_forward": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "hga_forward_causal": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "hga_stage_history": (ctypes.c_int, [_SHAPE, _P, _P, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P]),
    "hga_stage_history_min": (ctypes.c_int64, [_SHAPE, _I64, _I64]),
    "hga_attend_bwd_workspace_size": (ctypes.c_size_t, [_SHAPE, _I64, _I64]),
    "hga_attend_bwd": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P,
                                      _P, ctypes.c_size_t, _P]),
    "hga_attend_bwd_timed": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P,
                                            _P, ctypes.c_size_t, _P, _P]),
    "hga_decode_workspace_size": (ctypes.c_size_t, [_SHAPE, _I64]),
    "hga_decode_step": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                       _P]),
    "hga_decode_route": (ctypes.c_int, [_SHAPE, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "hga_decode_attend": (ctypes.c_int, [_SHAPE, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                         _P]),
    "hga_decode_step_noalloc": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P]),
    "hga_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_long_context_hga_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise HgaError(fn, st, lib().hga_status_string(st).decode())


# ---------------------------------------------------------------- thin wrappers
# Each wrapper checks its tensors on the host (dtype, contiguity, device, element
# count implied by the shape and sizes) and then passes their device pointers.
_I32, _F32, _U8 = torch.int32, torch.float32, torch.uint8


def _dims(shape: HgaShape):
    return shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim


def _cache_checks(fn, shape, dev, t_cap, k_cache, v_cache, group_sum, chunk_sum, optional_sums=False):
    """K/V cache [B,Hkv,t_cap,d] and summary tables [B,Hkv,t_cap/8,d], [B,Hkv,t_cap/64,d]
    (k_cache / v_cache skipped when passed as False)."""
    B, _, Hkv, d = _dims(shape)
    ft = _float_dtype(shape)
    if k_cache is not False:
        _need(fn, "k_cache", k_cache, ft, B * Hkv * t_cap * d, dev)
    if v_cache is not False:
        _need(fn, "v_cache", v_cache, ft, B * Hkv * t_cap * d, dev)
    _need(fn, "group_sum", group_sum, ft, B * Hkv * (t_cap // 8) * d, dev, optional=optional_sums)
    _need(fn, "chunk_sum", chunk_sum, ft, B * Hkv * (t_cap // 64) * d, dev, optional=optional_sums)


def hga_build_summaries(shape: HgaShape, k_cache: torch.Tensor, t_cap: int, t_begin: int, t_end: int,
                        group_sum: torch.Tensor, chunk_sum: torch.Tensor, stream=None) -> None:
    fn = "hga_build_summaries"
    dev = _dev_of(k_cache, group_sum, chunk_sum)
    _cache_checks(fn, shape, dev, t_cap, k_cache, False, group_sum, chunk_sum)
    _check(fn, lib().hga_build_summaries(
        ctypes.byref(shape), _ptr(k_cache), t_cap, t_begin, t_end, _ptr(group_sum), _ptr(chunk_sum),
        _stream(stream)))


def _route_checks(fn, shape, dev, q, chunk_sum, group_sum, t_cap, seg_len, chunk_idx, group_idx, chunk_score,
                  group_score):
    B, Hq, Hkv, d = _dims(shape)
    nb = seg_len // 64
    _need(fn, "q", q, _float_dtype(shape), B * Hq * seg_len * d, dev)
    _cache_checks(fn, shape, dev, t_cap, False, False, group_sum, chunk_sum)
    _need(fn, "chunk_idx", chunk_idx, _I32, B * Hkv * nb * shape.top_chunks, dev, optional=shape.top_chunks == 0)
    _need(fn, "group_idx", group_idx, _I32, B * Hkv * nb * shape.top_groups, dev, optional=shape.top_groups == 0)
    _need(fn, "chunk_score", chunk_score, _F32, B * Hkv * nb * shape.top_chunks, dev, optional=True)
    _need(fn, "group_score", group_score, _F32, B * Hkv * nb * shape.top_groups, dev, optional=True)


def hga_route(shape: HgaShape, q: torch.Tensor, chunk_sum: torch.Tensor, group_sum: torch.Tensor,
              t_cap: int, t_hist: int, seg_len: int, chunk_idx: torch.Tensor, group_idx: torch.Tensor,
              chunk_score: Optional[torch.Tensor] = None, group_score: Optional[torch.Tensor] = None,
              stream=None) -> None:
    fn = "hga_route"
    dev = _dev_of(q, chunk_sum, group_sum)
    _route_checks(fn, shape, dev, q, chunk_sum, group_sum, t_cap, seg_len, chunk_idx, group_idx, chunk_score,
                  group_score)
    _check(fn, lib().hga_route(
        ctypes.byref(shape), _ptr(q), _ptr(chunk_sum), _ptr(group_sum), t_cap, t_hist, seg_len,
        _ptr(chunk_idx), _ptr(group_idx), _ptr(chunk_score), _ptr(group_score), _stream(stream)))


def hga_route_causal(shape: HgaShape, q: torch.Tensor, q_prev: Optional[torch.Tensor], chunk_sum: torch.Tensor,
                     group_sum: torch.Tensor, t_cap: int, t_hist: int, seg_len: int, chunk_idx: torch.Tensor,
                     group_idx: torch.Tensor, chunk_score: Optional[torch.Tensor] = None,
                     group_score: Optional[torch.Tensor] = None, stream=None) -> None:
    fn = "hga_route_causal"
    dev = _dev_of(q, chunk_sum, group_sum)
    _route_checks(fn, shape, dev, q, chunk_sum, group_sum, t_cap, seg_len, chunk_idx, group_idx, chunk_score,
                  group_score)
    B, Hq, _, d = _dims(shape)
    _need(fn, "q_prev", q_prev, _float_dtype(shape), B * Hq * 64 * d, dev, optional=t_hist == 0)
    _check(fn, lib().hga_route_causal(
        ctypes.byref(shape), _ptr(q), _ptr(q_prev), _ptr(chunk_sum), _ptr(group_sum), t_cap, t_hist, seg_len,
        _ptr(chunk_idx), _ptr(group_idx), _ptr(chunk_score), _ptr(group_score), _stream(stream)))


def _attend_checks(fn, shape, dev, q, k_cache, v_cache, t_cap, seg_len, group_idx, o, lse):
    B, Hq, Hkv, d = _dims(shape)
    ft = _float_dtype(shape)
    _need(fn, "q", q, ft, B * Hq * seg_len * d, dev)
    _need(fn, "k_cache", k_cache, ft, B * Hkv * t_cap * d, dev)
    _need(fn, "v_cache", v_cache, ft, B * Hkv * t_cap * d, dev)
    _need(fn, "group_idx", group_idx, _I32, B * Hkv * (seg_len // 64) * shape.top_groups, dev,
          optional=shape.top_groups == 0)
    _need(fn, "o", o, ft, B * Hq * seg_len * d, dev)
    _need(fn, "lse", lse, _F32, B * Hq * seg_len, dev)


def hga_attend_fwd(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   t_cap: int, t_hist: int, seg_len: int, group_idx: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, stream=None) -> None:
    fn = "hga_attend_fwd"
    dev = _dev_of(q, k_cache, v_cache)
    _attend_checks(fn, shape, dev, q, k_cache, v_cache, t_cap, seg_len, group_idx, o, lse)
    _check(fn, lib().hga_attend_fwd(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, t_hist, seg_len,
        _ptr(group_idx), _ptr(o), _ptr(lse), _stream(stream)))


HGA_FWD_EVENTS = 4


def _event_handles(events, n, stream):
    """ctypes array of n HIP event handles from torch.cuda.Event objects (None
    entries stay NULL); torch creates an event's HIP handle on its first record."""
    if len(events) != n:
        raise ValueError(f"need {n} events, got {len(events)}")
    for e in events:
        if e is not None and not e.cuda_event:
            e.record(stream if stream is not None else torch.cuda.current_stream())
    return (ctypes.c_void_p * n)(*[None if e is None else ctypes.c_void_p(e.cuda_event) for e in events])


def hga_forward(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                chunk_sum: torch.Tensor, group_sum: torch.Tensor, t_cap: int, t_hist: int, seg_len: int,
                chunk_idx: Optional[torch.Tensor], group_idx: Optional[torch.Tensor], o: torch.Tensor,
                lse: torch.Tensor, events=None, stream=None) -> None:
    """Summaries of the active segment, routing and attention in one call (events:
    None or HGA_FWD_EVENTS torch.cuda.Event / None entries, recorded by the dispatches)."""
    fn = "hga_forward"
    dev = _dev_of(q, k_cache, v_cache)
    _route_checks(fn, shape, dev, q, chunk_sum, group_sum, t_cap, seg_len, chunk_idx, group_idx, None, None)
    _attend_checks(fn, shape, dev, q, k_cache, v_cache, t_cap, seg_len, group_idx, o, lse)
    handles = None if events is None else _event_handles(events, HGA_FWD_EVENTS, stream)
    _check(fn, lib().hga_forward(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(chunk_sum), _ptr(group_sum), t_cap, t_hist,
        seg_len, _ptr(chunk_idx), _ptr(group_idx), _ptr(o), _ptr(lse), handles, _stream(stream)))


def hga_forward_causal(shape: HgaShape, q: torch.Tensor, q_prev: Optional[torch.Tensor], k_cache: torch.Tensor,
                       v_cache: torch.Tensor, chunk_sum: torch.Tensor, group_sum: torch.Tensor, t_cap: int,
                       t_hist: int, seg_len: int, chunk_idx: Optional[torch.Tensor], group_idx: Optional[torch.Tensor],
                       o: torch.Tensor, lse: torch.Tensor, events=None, stream=None) -> None:
    """hga_forward with strictly causal routing (each block routed by the block before
    it, q_prev [B, Hq, 64, d] for the first; needed when t_hist > 0)."""
    fn = "hga_forward_causal"
    dev = _dev_of(q, k_cache, v_cache)
    _route_checks(fn, shape, dev, q, chunk_sum, group_sum, t_cap, seg_len, chunk_idx, group_idx, None, None)
    _attend_checks(fn, shape, dev, q, k_cache, v_cache, t_cap, seg_len, group_idx, o, lse)
    B, Hq, _, d = _dims(shape)
    _need(fn, "q_prev", q_prev, _float_dtype(shape), B * Hq * 64 * d, dev, optional=t_hist == 0)
    handles = None if events is None else _event_handles(events, HGA_FWD_EVENTS, stream)
    _check(fn, lib().hga_forward_causal(
        ctypes.byref(shape), _ptr(q), _ptr(q_prev), _ptr(k_cache), _ptr(v_cache), _ptr(chunk_sum), _ptr(group_sum),
        t_cap, t_hist, seg_len, _ptr(chunk_idx), _ptr(group_idx), _ptr(o), _ptr(lse), handles, _stream(stream)))


def hga_stage_history_min(shape: HgaShape, t_hist: int, seg_len: int) -> int:
    return int(lib().hga_stage_history_min(ctypes.byref(shape), t_hist, seg_len))


def hga_stage_history(shape: HgaShape, k_host: torch.Tensor, v_host: torch.Tensor, host_t_cap: int, t_hist: int,
                      seg_len: int, group_idx: torch.Tensor, k_stage: torch.Tensor, v_stage: torch.Tensor,
                      stage_cap: int, stage_hist: int, group_idx_stage: torch.Tensor, stream=None) -> None:
    """Copy the selected history groups from pinned host memory into the staging cache
    and renumber the selection for it (the host-RAM history tier)."""
    fn = "hga_stage_history"
    dev = _dev_of(k_stage, v_stage)
    B, _, Hkv, d = _dims(shape)
    ft = _float_dtype(shape)
    for name, t in (("k_host", k_host), ("v_host", v_host)):
        _need(fn, name, t, ft, B * Hkv * host_t_cap * d, None)
        if t.device.type != "cpu" or not t.is_pinned():
            raise ValueError(f"{fn}: {name} must be pinned host memory")
    _need(fn, "k_stage", k_stage, ft, B * Hkv * stage_cap * d, dev)
    _need(fn, "v_stage", v_stage, ft, B * Hkv * stage_cap * d, dev)
    n_ids = B * Hkv * (seg_len // 64) * shape.top_groups
    _need(fn, "group_idx", group_idx, _I32, n_ids, dev, optional=shape.top_groups == 0)
    _need(fn, "group_idx_stage", group_idx_stage, _I32, n_ids, dev, optional=shape.top_groups == 0)
    _check(fn, lib().hga_stage_history(
        ctypes.byref(shape), _ptr(k_host), _ptr(v_host), host_t_cap, t_hist, seg_len, _ptr(group_idx), _ptr(k_stage),
        _ptr(v_stage), stage_cap, stage_hist, _ptr(group_idx_stage), _stream(stream)))


def hga_attend_bwd_workspace_size(shape: HgaShape, t_hist: int, seg_len: int) -> int:
    return int(lib().hga_attend_bwd_workspace_size(ctypes.byref(shape), t_hist, seg_len))


def _bwd_checks(fn, shape, dev, q, k_cache, v_cache, o, lse, d_o, t_cap, seg_len, group_idx, dq, dk_active,
                dv_active, workspace):
    B, Hq, Hkv, d = _dims(shape)
    ft = _float_dtype(shape)
    _attend_checks(fn, shape, dev, q, k_cache, v_cache, t_cap, seg_len, group_idx, o, lse)
    _need(fn, "d_o", d_o, ft, B * Hq * seg_len * d, dev)
    _need(fn, "dq", dq, ft, B * Hq * seg_len * d, dev)
    _need(fn, "dk_active", dk_active, ft, B * Hkv * seg_len * d, dev)
    _need(fn, "dv_active", dv_active, ft, B * Hkv * seg_len * d, dev)
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"{fn}: workspace must be a contiguous tensor on {dev}")


def hga_attend_bwd(shape: HgaShape, q, k_cache, v_cache, o, lse, d_o, t_cap: int, t_hist: int,
                   seg_len: int, group_idx, dq, dk_active, dv_active, workspace: torch.Tensor,
                   stream=None) -> None:
    fn = "hga_attend_bwd"
    dev = _dev_of(q, k_cache, v_cache)
    _bwd_checks(fn, shape, dev, q, k_cache, v_cache, o, lse, d_o, t_cap, seg_len, group_idx, dq, dk_active,
                dv_active, workspace)
    _check(fn, lib().hga_attend_bwd(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(d_o),
        t_cap, t_hist, seg_len, _ptr(group_idx), _ptr(dq), _ptr(dk_active), _ptr(dv_active),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


HGA_BWD_KERNELS = 3
HGA_BWD_WORKSPACE_CLEAR_BYTES = 256   # leading workspace bytes that must be zero before first use


def hga_attend_bwd_timed(shape: HgaShape, q, k_cache, v_cache, o, lse, d_o, t_cap: int, t_hist: int,
                         seg_len: int, group_idx, dq, dk_active, dv_active, workspace: torch.Tensor,
                         events, stream=None) -> None:
    """hga_attend_bwd with torch.cuda.Event pairs recorded around each of its kernels
    (events[2i], events[2i+1] for kernel i; None entries are skipped)."""
    fn = "hga_attend_bwd_timed"
    if len(events) != 2 * HGA_BWD_KERNELS:
        raise ValueError(f"need {2 * HGA_BWD_KERNELS} events, got {len(events)}")
    dev = _dev_of(q, k_cache, v_cache)
    _bwd_checks(fn, shape, dev, q, k_cache, v_cache, o, lse, d_o, t_cap, seg_len, group_idx, dq, dk_active,
                dv_active, workspace)
    handles = _event_handles(events, 2 * HGA_BWD_KERNELS, stream)
    _check(fn, lib().hga_attend_bwd_timed(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(d_o),
        t_cap, t_hist, seg_len, _ptr(group_idx), _ptr(dq), _ptr(dk_active), _ptr(dv_active),
        _ptr(workspace), _nbytes(workspace), handles, _stream(stream)))


def hga_decode_workspace_size(shape: HgaShape, t_cap: int) -> int:
    return int(lib().hga_decode_workspace_size(ctypes.byref(shape), t_cap))


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _decode_checks(fn, shape, dev, q, t_cap, pos, chunk_idx, group_idx, workspace, chunk_optional=False):
    B, Hq, Hkv, d = _dims(shape)
    _need(fn, "q", q, _float_dtype(shape), B * Hq * d, dev)
    _need(fn, "pos", pos, _I32, B, dev)
    _need(fn, "chunk_idx", chunk_idx, _I32, B * Hkv * shape.top_chunks, dev,
          optional=chunk_optional or shape.top_chunks == 0)
    _need(fn, "group_idx", group_idx, _I32, B * Hkv * shape.top_groups, dev, optional=shape.top_groups == 0)
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.device != dev
                                  or not workspace.is_contiguous()):
        raise ValueError(f"{fn}: workspace must be a contiguous tensor on {dev}")


def hga_decode_step(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    chunk_sum: torch.Tensor, group_sum: torch.Tensor, t_cap: int, pos: torch.Tensor,
                    chunk_idx: Optional[torch.Tensor], group_idx: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    fn = "hga_decode_step"
    dev = _dev_of(q, k_cache, v_cache)
    B, Hq, _, d = _dims(shape)
    _decode_checks(fn, shape, dev, q, t_cap, pos, chunk_idx, group_idx, workspace, chunk_optional=True)
    _cache_checks(fn, shape, dev, t_cap, k_cache, v_cache, group_sum, chunk_sum)
    _need(fn, "o", o, _float_dtype(shape), B * Hq * d, dev)
    _need(fn, "lse", lse, _F32, B * Hq, dev)
    _check(fn, lib().hga_decode_step(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(chunk_sum), _ptr(group_sum), t_cap,
        _ptr(pos), _ptr(chunk_idx), _ptr(group_idx), _ptr(o), _ptr(lse), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def hga_decode_step_noalloc(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            chunk_sum: torch.Tensor, group_sum: torch.Tensor, t_cap: int, pos: torch.Tensor,
                            chunk_idx: Optional[torch.Tensor], group_idx: torch.Tensor, o: torch.Tensor,
                            lse: torch.Tensor, stream=None) -> None:
    """hga_decode_step with the library's static device scratch as its workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    fn = "hga_decode_step_noalloc"
    dev = _dev_of(q, k_cache, v_cache)
    B, Hq, _, d = _dims(shape)
    _decode_checks(fn, shape, dev, q, t_cap, pos, chunk_idx, group_idx, None, chunk_optional=True)
    _cache_checks(fn, shape, dev, t_cap, k_cache, v_cache, group_sum, chunk_sum)
    _need(fn, "o", o, _float_dtype(shape), B * Hq * d, dev)
    _need(fn, "lse", lse, _F32, B * Hq, dev)
    _check(fn, lib().hga_decode_step_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(chunk_sum), _ptr(group_sum), t_cap,
        _ptr(pos), _ptr(chunk_idx), _ptr(group_idx), _ptr(o), _ptr(lse), _stream(stream)))


def hga_decode_route(shape: HgaShape, q: torch.Tensor, chunk_sum: torch.Tensor, group_sum: torch.Tensor,
                     t_cap: int, pos: torch.Tensor, chunk_idx: torch.Tensor, group_idx: torch.Tensor,
                     workspace: torch.Tensor, chunk_score: Optional[torch.Tensor] = None,
                     group_score: Optional[torch.Tensor] = None, stream=None) -> None:
    fn = "hga_decode_route"
    dev = _dev_of(q, chunk_sum, group_sum)
    B, _, Hkv, d = _dims(shape)
    _decode_checks(fn, shape, dev, q, t_cap, pos, chunk_idx, group_idx, workspace)
    _cache_checks(fn, shape, dev, t_cap, False, False, group_sum, chunk_sum)
    _need(fn, "chunk_score", chunk_score, _F32, B * Hkv * shape.top_chunks, dev, optional=True)
    _need(fn, "group_score", group_score, _F32, B * Hkv * shape.top_groups, dev, optional=True)
    _check(fn, lib().hga_decode_route(
        ctypes.byref(shape), _ptr(q), _ptr(chunk_sum), _ptr(group_sum), t_cap, _ptr(pos), _ptr(chunk_idx),
        _ptr(group_idx), _ptr(chunk_score), _ptr(group_score), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def hga_decode_attend(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      t_cap: int, pos: torch.Tensor, group_idx: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                      workspace: torch.Tensor, group_sum: Optional[torch.Tensor] = None,
                      chunk_sum: Optional[torch.Tensor] = None, stream=None) -> None:
    fn = "hga_decode_attend"
    dev = _dev_of(q, k_cache, v_cache)
    B, Hq, _, d = _dims(shape)
    _decode_checks(fn, shape, dev, q, t_cap, pos, None, group_idx, workspace, chunk_optional=True)
    _cache_checks(fn, shape, dev, t_cap, k_cache, v_cache, group_sum, chunk_sum, optional_sums=True)
    _need(fn, "o", o, _float_dtype(shape), B * Hq * d, dev)
    _need(fn, "lse", lse, _F32, B * Hq, dev)
    _check(fn, lib().hga_decode_attend(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, _ptr(pos), _ptr(group_idx), _ptr(o),
        _ptr(lse), _ptr(group_sum), _ptr(chunk_sum), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def hga_status_string(status: int) -> str:
    return lib().hga_status_string(status).decode()


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
