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


def make_shape(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, top_chunks: int,
               top_groups: int, dtype: str = "bf16", softmax_scale: float = 0.0) -> HgaShape:
    return HgaShape(batch, n_q_heads, n_kv_heads, head_dim, 64, 8, 64, top_chunks, top_groups,
                    HGA_BF16 if dtype == "bf16" else HGA_F32, softmax_scale)


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SHAPE = ctypes.POINTER(HgaShape)

SIGNATURES = {
    "hga_build_summaries": (ctypes.c_int, [_SHAPE, _P, _I64, _I64, _I64, _P, _P, _P]),
    "hga_route": (ctypes.c_int, [_SHAPE, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "hga_route_causal": (ctypes.c_int, [_SHAPE, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "hga_attend_fwd": (ctypes.c_int, [_SHAPE, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
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
def hga_build_summaries(shape: HgaShape, k_cache: torch.Tensor, t_cap: int, t_begin: int, t_end: int,
                        group_sum: torch.Tensor, chunk_sum: torch.Tensor, stream=None) -> None:
    _check("hga_build_summaries", lib().hga_build_summaries(
        ctypes.byref(shape), _ptr(k_cache), t_cap, t_begin, t_end, _ptr(group_sum), _ptr(chunk_sum),
        _stream(stream)))


def hga_route(shape: HgaShape, q: torch.Tensor, chunk_sum: torch.Tensor, group_sum: torch.Tensor,
              t_cap: int, t_hist: int, seg_len: int, chunk_idx: torch.Tensor, group_idx: torch.Tensor,
              chunk_score: Optional[torch.Tensor] = None, group_score: Optional[torch.Tensor] = None,
              stream=None) -> None:
    _check("hga_route", lib().hga_route(
        ctypes.byref(shape), _ptr(q), _ptr(chunk_sum), _ptr(group_sum), t_cap, t_hist, seg_len,
        _ptr(chunk_idx), _ptr(group_idx), _ptr(chunk_score), _ptr(group_score), _stream(stream)))


def hga_route_causal(shape: HgaShape, q: torch.Tensor, q_prev: Optional[torch.Tensor], chunk_sum: torch.Tensor,
                     group_sum: torch.Tensor, t_cap: int, t_hist: int, seg_len: int, chunk_idx: torch.Tensor,
                     group_idx: torch.Tensor, chunk_score: Optional[torch.Tensor] = None,
                     group_score: Optional[torch.Tensor] = None, stream=None) -> None:
    _check("hga_route_causal", lib().hga_route_causal(
        ctypes.byref(shape), _ptr(q), _ptr(q_prev), _ptr(chunk_sum), _ptr(group_sum), t_cap, t_hist, seg_len,
        _ptr(chunk_idx), _ptr(group_idx), _ptr(chunk_score), _ptr(group_score), _stream(stream)))


def hga_attend_fwd(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   t_cap: int, t_hist: int, seg_len: int, group_idx: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, stream=None) -> None:
    _check("hga_attend_fwd", lib().hga_attend_fwd(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, t_hist, seg_len,
        _ptr(group_idx), _ptr(o), _ptr(lse), _stream(stream)))


def hga_attend_bwd_workspace_size(shape: HgaShape, t_hist: int, seg_len: int) -> int:
    return int(lib().hga_attend_bwd_workspace_size(ctypes.byref(shape), t_hist, seg_len))


def hga_attend_bwd(shape: HgaShape, q, k_cache, v_cache, o, lse, d_o, t_cap: int, t_hist: int,
                   seg_len: int, group_idx, dq, dk_active, dv_active, workspace: torch.Tensor,
                   stream=None) -> None:
    _check("hga_attend_bwd", lib().hga_attend_bwd(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(d_o),
        t_cap, t_hist, seg_len, _ptr(group_idx), _ptr(dq), _ptr(dk_active), _ptr(dv_active),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


HGA_BWD_KERNELS = 4


def hga_attend_bwd_timed(shape: HgaShape, q, k_cache, v_cache, o, lse, d_o, t_cap: int, t_hist: int,
                         seg_len: int, group_idx, dq, dk_active, dv_active, workspace: torch.Tensor,
                         events, stream=None) -> None:
    """hga_attend_bwd with torch.cuda.Event pairs recorded around each of its kernels
    (events[2i], events[2i+1] for kernel i; None entries are skipped)."""
    if len(events) != 2 * HGA_BWD_KERNELS:
        raise ValueError(f"need {2 * HGA_BWD_KERNELS} events, got {len(events)}")
    for e in events:
        if e is not None and not e.cuda_event:
            e.record(stream if stream is not None else torch.cuda.current_stream())  # creates it
    handles = (ctypes.c_void_p * (2 * HGA_BWD_KERNELS))(
        *[None if e is None else ctypes.c_void_p(e.cuda_event) for e in events])
    _check("hga_attend_bwd_timed", lib().hga_attend_bwd_timed(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(d_o),
        t_cap, t_hist, seg_len, _ptr(group_idx), _ptr(dq), _ptr(dk_active), _ptr(dv_active),
        _ptr(workspace), workspace.numel() * workspace.element_size(), handles, _stream(stream)))


def hga_decode_workspace_size(shape: HgaShape, t_cap: int) -> int:
    return int(lib().hga_decode_workspace_size(ctypes.byref(shape), t_cap))


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def hga_decode_step(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    chunk_sum: torch.Tensor, group_sum: torch.Tensor, t_cap: int, pos: torch.Tensor,
                    chunk_idx: Optional[torch.Tensor], group_idx: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    _check("hga_decode_step", lib().hga_decode_step(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(chunk_sum), _ptr(group_sum), t_cap,
        _ptr(pos), _ptr(chunk_idx), _ptr(group_idx), _ptr(o), _ptr(lse), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def hga_decode_route(shape: HgaShape, q: torch.Tensor, chunk_sum: torch.Tensor, group_sum: torch.Tensor,
                     t_cap: int, pos: torch.Tensor, chunk_idx: torch.Tensor, group_idx: torch.Tensor,
                     workspace: torch.Tensor, chunk_score: Optional[torch.Tensor] = None,
                     group_score: Optional[torch.Tensor] = None, stream=None) -> None:
    _check("hga_decode_route", lib().hga_decode_route(
        ctypes.byref(shape), _ptr(q), _ptr(chunk_sum), _ptr(group_sum), t_cap, _ptr(pos), _ptr(chunk_idx),
        _ptr(group_idx), _ptr(chunk_score), _ptr(group_score), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def hga_decode_attend(shape: HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      t_cap: int, pos: torch.Tensor, group_idx: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                      workspace: torch.Tensor, group_sum: Optional[torch.Tensor] = None,
                      chunk_sum: Optional[torch.Tensor] = None, stream=None) -> None:
    _check("hga_decode_attend", lib().hga_decode_attend(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, _ptr(pos), _ptr(group_idx), _ptr(o),
        _ptr(lse), _ptr(group_sum), _ptr(chunk_sum), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def hga_status_string(status: int) -> str:
    return lib().hga_status_string(status).decode()


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
