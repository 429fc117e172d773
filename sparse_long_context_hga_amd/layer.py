"""Device-side state and the layer step built on the four library calls.

Everything here is plumbing: PyTorch allocates device memory and provides the
stream; every step of the computation runs in libhga.so.

  HGALayerBuffers  -- the buffers of one routed-attention layer step (cache,
                      summaries, selection, outputs, gradients, workspace) and
                      the calls in hot-path order.
  HGAKVCache       -- a per-layer K/V cache with its summary tables that grows
                      segment by segment (segment-wise training and rollout).
  hga_attention    -- autograd op for one active segment: forward routes and
                      attends; backward returns dQ, dK, dV of the active segment
                      only (the history is detached).
  HGADecoder       -- generation over an HGAKVCache: one new token per sequence
                      per step (per-token routing, attention, and the summaries of
                      a chunk once its last token is in).
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib as L


def _dt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _dtype_name(t: torch.dtype) -> str:
    if t == torch.bfloat16:
        return "bf16"
    if t == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t}")


class HGALayerBuffers:
    """Buffers of one layer step on the current device.

    q [B,Hq,S,d]; k_cache/v_cache [B,Hkv,t_cap,d] (history at [0,t_hist), the
    active segment after it); optional d_o [B,Hq,S,d] for the backward.
    """

    def __init__(self, shape: L.HgaShape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 t_hist: int, d_o: Optional[torch.Tensor] = None):
        self.shape = shape
        self.q, self.k, self.v, self.do = q, k_cache, v_cache, d_o
        B, Hq, S, d = q.shape
        Hkv, t_cap = k_cache.shape[1], k_cache.shape[2]
        self.t_hist, self.seg_len, self.t_cap = t_hist, S, t_cap
        dev, dt = q.device, q.dtype
        nb = S // 64
        kc, kg = shape.top_chunks, shape.top_groups
        self.gsum = torch.zeros(B, Hkv, t_cap // 8, d, dtype=dt, device=dev)
        self.csum = torch.zeros(B, Hkv, t_cap // 64, d, dtype=dt, device=dev)
        self.cidx = torch.empty(B, Hkv, nb, kc, dtype=torch.int32, device=dev)
        self.gidx = torch.empty(B, Hkv, nb, kg, dtype=torch.int32, device=dev)
        self.cscore = torch.empty(B, Hkv, nb, kc, dtype=torch.float32, device=dev)
        self.gscore = torch.empty(B, Hkv, nb, kg, dtype=torch.float32, device=dev)
        self.o = torch.empty_like(q)
        self.lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(q)
        self.dk = torch.empty(B, Hkv, S, d, dtype=dt, device=dev)
        self.dv = torch.empty(B, Hkv, S, d, dtype=dt, device=dev)
        ws = L.hga_attend_bwd_workspace_size(shape, t_hist, S)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)

    def summaries(self, t_begin: int, t_end: int):
        L.hga_build_summaries(self.shape, self.k, self.t_cap, t_begin, t_end, self.gsum, self.csum)

    def route(self, csum: Optional[torch.Tensor] = None, gsum: Optional[torch.Tensor] = None):
        L.hga_route(self.shape, self.q, self.csum if csum is None else csum,
                    self.gsum if gsum is None else gsum, self.t_cap, self.t_hist, self.seg_len,
                    self.cidx, self.gidx, self.cscore, self.gscore)

    def route_causal(self, q_prev: Optional[torch.Tensor], csum: Optional[torch.Tensor] = None,
                     gsum: Optional[torch.Tensor] = None):
        """Strictly causal routing: block j routed by block j-1 (q_prev for the first block)."""
        L.hga_route_causal(self.shape, self.q, q_prev, self.csum if csum is None else csum,
                           self.gsum if gsum is None else gsum, self.t_cap, self.t_hist, self.seg_len,
                           self.cidx, self.gidx, self.cscore, self.gscore)

    def fwd(self, gidx: Optional[torch.Tensor] = None):
        L.hga_attend_fwd(self.shape, self.q, self.k, self.v, self.t_cap, self.t_hist, self.seg_len,
                         self.gidx if gidx is None else gidx, self.o, self.lse)

    def bwd(self, gidx: Optional[torch.Tensor] = None, events=None):
        g = self.gidx if gidx is None else gidx
        if events is None:
            L.hga_attend_bwd(self.shape, self.q, self.k, self.v, self.o, self.lse, self.do, self.t_cap,
                             self.t_hist, self.seg_len, g, self.dq, self.dk, self.dv, self.ws)
        else:
            L.hga_attend_bwd_timed(self.shape, self.q, self.k, self.v, self.o, self.lse, self.do, self.t_cap,
                                   self.t_hist, self.seg_len, g, self.dq, self.dk, self.dv, self.ws, events)

    def step(self):
        """One pass of the hot path: active-segment summaries, route, forward, backward."""
        self.summaries(self.t_hist, self.t_hist + self.seg_len)
        self.route()
        self.fwd()
        if self.do is not None:
            self.bwd()


class HGAKVCache:
    """K/V of one layer for `batch` sequences, with group/chunk summary tables.

    Positions [0, length) are written; appending a segment writes its K/V and
    summaries.  Gradients never flow into the cache: a segment's K/V become
    detached history once the next segment starts.  For strictly causal routing
    the cache also keeps the last query block of the latest committed segment
    (it routes the next segment's first block).
    """

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, t_cap: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda"):
        if t_cap % 64:
            raise ValueError("t_cap must be a multiple of 64")
        self.batch, self.n_kv_heads, self.head_dim, self.t_cap = batch, n_kv_heads, head_dim, t_cap
        self.dtype = dtype
        self.k = torch.zeros(batch, n_kv_heads, t_cap, head_dim, dtype=dtype, device=device)
        self.v = torch.zeros_like(self.k)
        self.gsum = torch.zeros(batch, n_kv_heads, t_cap // 8, head_dim, dtype=dtype, device=device)
        self.csum = torch.zeros(batch, n_kv_heads, t_cap // 64, head_dim, dtype=dtype, device=device)
        self.length = 0
        self.q_last: Optional[torch.Tensor] = None      # [B, Hq, 64, d] of the committed history
        self._q_pending: Optional[torch.Tensor] = None

    def write(self, k_seg: torch.Tensor, v_seg: torch.Tensor, shape: L.HgaShape) -> int:
        """Place a segment's K/V at [length, length+S) and build its summaries.
        Returns the position where it starts (the history length for the segment)."""
        S = k_seg.shape[2]
        t0 = self.length
        if t0 + S > self.t_cap:
            raise ValueError("KV cache capacity exceeded")
        self.k[:, :, t0:t0 + S].copy_(k_seg.detach())
        self.v[:, :, t0:t0 + S].copy_(v_seg.detach())
        L.hga_build_summaries(shape, self.k, self.t_cap, t0, t0 + S, self.gsum, self.csum)
        return t0

    def keep_last_query_block(self, q: torch.Tensor):
        """Remember the written segment's last 64 query rows (taken over by commit)."""
        self._q_pending = q[:, :, -64:].detach().contiguous().clone()

    def commit(self, seg_len: int):
        """The written segment becomes history."""
        self.length += seg_len
        self.q_last, self._q_pending = self._q_pending, None


class _HGAAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k_seg, v_seg, cache: HGAKVCache, top_chunks: int, top_groups: int, scale: float,
                causal_routing: bool):
        B, Hq, S, d = q.shape
        shape = L.make_shape(B, Hq, cache.n_kv_heads, d, top_chunks, top_groups, _dtype_name(q.dtype), scale)
        q = q.contiguous()
        if causal_routing and cache.length > 0 and (cache.q_last is None or cache.q_last.shape[1] != Hq):
            raise ValueError("causal routing over history needs the previous segment's last query block "
                             "(route every segment of the cache causally)")
        t_hist = cache.write(k_seg, v_seg, shape)
        nb = S // 64
        cidx = torch.empty(B, cache.n_kv_heads, nb, top_chunks, dtype=torch.int32, device=q.device)
        gidx = torch.empty(B, cache.n_kv_heads, nb, top_groups, dtype=torch.int32, device=q.device)
        if causal_routing:
            L.hga_route_causal(shape, q, cache.q_last if t_hist > 0 else None, cache.csum, cache.gsum,
                               cache.t_cap, t_hist, S, cidx, gidx)
        else:
            L.hga_route(shape, q, cache.csum, cache.gsum, cache.t_cap, t_hist, S, cidx, gidx)
        cache.keep_last_query_block(q)
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
        L.hga_attend_fwd(shape, q, cache.k, cache.v, cache.t_cap, t_hist, S, gidx, o, lse)
        ctx.save_for_backward(q, o, lse, gidx)
        ctx.cache, ctx.shape, ctx.t_hist = cache, shape, t_hist
        ctx.mark_non_differentiable(gidx)
        return o, gidx

    @staticmethod
    def backward(ctx, d_o, _g):
        q, o, lse, gidx = ctx.saved_tensors
        cache, shape, t_hist = ctx.cache, ctx.shape, ctx.t_hist
        B, Hq, S, d = q.shape
        dq = torch.empty_like(q)
        dk = torch.empty(B, cache.n_kv_heads, S, d, dtype=q.dtype, device=q.device)
        dv = torch.empty_like(dk)
        ws = torch.empty(max(L.hga_attend_bwd_workspace_size(shape, t_hist, S), 16), dtype=torch.uint8,
                         device=q.device)
        L.hga_attend_bwd(shape, q, cache.k, cache.v, o, lse, d_o.contiguous(), cache.t_cap, t_hist, S, gidx,
                         dq, dk, dv, ws)
        return dq, dk, dv, None, None, None, None, None


def hga_attention(q: torch.Tensor, k_seg: torch.Tensor, v_seg: torch.Tensor, cache: HGAKVCache,
                  top_chunks: int = 16, top_groups: int = 64, softmax_scale: Optional[float] = None,
                  causal_routing: bool = False):
    """Routed attention of one active segment against the cache's history plus itself.

    q [B,Hq,S,d], k_seg/v_seg [B,Hkv,S,d] (the segment's keys/values, written into
    the cache at its current length).  Returns (o [B,Hq,S,d], group_idx).  Call
    cache.commit(S) once the segment's backward is done to turn it into history.
    causal_routing: route each block with the block before it (hga_route_causal);
    then every segment written to the cache must be routed that way.
    """
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    return _HGAAttentionFn.apply(q, k_seg, v_seg, cache, top_chunks, top_groups, scale, causal_routing)


class HGADecoder:
    """Generation steps over `cache`: every sequence adds one token per step.

    step(q, k_new, v_new, pos) writes the new tokens' K/V at positions pos (a [B]
    int32 device tensor; a negative entry marks an idle slot), routes each token
    with its own query heads, attends, and builds the summaries of every chunk
    whose last token this step wrote.  Returns (o [B,Hq,d], lse [B,Hq], group_idx).
    The cache's `length` is not used: positions come from `pos`.
    """

    def __init__(self, cache: HGAKVCache, n_q_heads: int, top_chunks: int = 16, top_groups: int = 64,
                 softmax_scale: Optional[float] = None):
        B, Hkv, d = cache.batch, cache.n_kv_heads, cache.head_dim
        dev = cache.k.device
        scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
        self.cache = cache
        self.shape = L.make_shape(B, n_q_heads, Hkv, d, top_chunks, top_groups, _dtype_name(cache.dtype), scale)
        self.cidx = torch.empty(B, Hkv, top_chunks, dtype=torch.int32, device=dev)
        self.gidx = torch.empty(B, Hkv, top_groups, dtype=torch.int32, device=dev)
        self.o = torch.empty(B, n_q_heads, d, dtype=cache.dtype, device=dev)
        self.lse = torch.empty(B, n_q_heads, dtype=torch.float32, device=dev)
        self.ws = torch.zeros(L.hga_decode_workspace_size(self.shape, cache.t_cap), dtype=torch.uint8, device=dev)
        self._b = torch.arange(B, device=dev)

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor):
        c = self.cache
        live = pos >= 0
        bi, p = self._b[live], pos[live].long()
        c.k[bi, :, p] = k_new[live].to(c.dtype)
        c.v[bi, :, p] = v_new[live].to(c.dtype)
        L.hga_decode_step(self.shape, q.contiguous(), c.k, c.v, c.csum, c.gsum, c.t_cap, pos, self.cidx,
                          self.gidx, self.o, self.lse, self.ws)
        return self.o, self.lse, self.gidx
