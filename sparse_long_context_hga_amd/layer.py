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
  HGAHostKVCache   -- the same with the detached history's K/V in pinned host
                      memory (host-RAM tier): HBM holds the summary tables, the
                      active segment and a staging cache for the selected groups.
  HGAStack         -- segment-wise truncated backpropagation through a stack of
                      HGA layers, each with its own cache (forward, backward,
                      detach, next segment).
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
        self.ws = torch.empty(max(ws, L.HGA_BWD_WORKSPACE_CLEAR_BYTES), dtype=torch.uint8, device=dev)
        self.ws[:L.HGA_BWD_WORKSPACE_CLEAR_BYTES].zero_()     # every backward call leaves them zero

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

    def forward(self, events=None):
        """Summaries of the active segment, routing and attention in one call
        (hga_forward); events: None or HGA_FWD_EVENTS torch.cuda.Event entries."""
        L.hga_forward(self.shape, self.q, self.k, self.v, self.csum, self.gsum, self.t_cap, self.t_hist,
                      self.seg_len, self.cidx, self.gidx, self.o, self.lse, events)

    def forward_causal(self, q_prev: Optional[torch.Tensor], events=None):
        """hga_forward with strictly causal routing (hga_forward_causal): block j routed
        by block j-1, the first block by q_prev (needed when t_hist > 0)."""
        L.hga_forward_causal(self.shape, self.q, q_prev if self.t_hist > 0 else None, self.k, self.v, self.csum,
                             self.gsum, self.t_cap, self.t_hist, self.seg_len, self.cidx, self.gidx, self.o,
                             self.lse, events)

    def bwd(self, gidx: Optional[torch.Tensor] = None, events=None):
        g = self.gidx if gidx is None else gidx
        if events is None:
            L.hga_attend_bwd(self.shape, self.q, self.k, self.v, self.o, self.lse, self.do, self.t_cap,
                             self.t_hist, self.seg_len, g, self.dq, self.dk, self.dv, self.ws)
        else:
            L.hga_attend_bwd_timed(self.shape, self.q, self.k, self.v, self.o, self.lse, self.do, self.t_cap,
                                   self.t_hist, self.seg_len, g, self.dq, self.dk, self.dv, self.ws, events)

    def step(self):
        """One pass of the hot path: active-segment summaries, route and forward
        (hga_forward), then the backward."""
        self.forward()
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

    def write(self, k_seg: torch.Tensor, v_seg: torch.Tensor, shape: L.HgaShape, summaries: bool = True) -> int:
        """Place a segment's K/V at [length, length+S) and build its summaries (unless
        the caller builds them, as hga_forward does).  Returns the position where it
        starts (the history length for the segment)."""
        S = k_seg.shape[2]
        t0 = self.length
        if t0 + S > self.t_cap:
            raise ValueError("KV cache capacity exceeded")
        self.k[:, :, t0:t0 + S].copy_(k_seg.detach())
        self.v[:, :, t0:t0 + S].copy_(v_seg.detach())
        if summaries:
            L.hga_build_summaries(shape, self.k, self.t_cap, t0, t0 + S, self.gsum, self.csum)
        return t0

    def keep_last_query_block(self, q: torch.Tensor):
        """Remember the written segment's last 64 query rows (taken over by commit)."""
        self._q_pending = q[:, :, -64:].detach().contiguous().clone()

    def commit(self, seg_len: int):
        """The written segment becomes history."""
        self.length += seg_len
        self.q_last, self._q_pending = self._q_pending, None


class HGAHostKVCache:
    """K/V of one layer with the detached history in pinned host memory.

    HBM holds the group/chunk summary tables of the whole capacity (routing reads
    only those), the active segment, and a staging cache into which
    hga_stage_history copies, per segment, the history groups that the segment's
    query blocks selected.  Segments have a fixed length seg_len and a fixed
    budget (top_groups), which bound the staging cache: at most 8 * seg_len/64 *
    top_groups history tokens.  The attention runs on the staging cache with
    results bit-identical to HGAKVCache's; committing a segment copies its K/V
    to host memory.
    """

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, t_cap: int, seg_len: int, n_q_heads: int,
                 top_chunks: int, top_groups: int, dtype: torch.dtype = torch.bfloat16, device="cuda"):
        if t_cap % 64 or seg_len % 64 or seg_len <= 0:
            raise ValueError("t_cap and seg_len must be multiples of 64")
        self.batch, self.n_kv_heads, self.head_dim, self.t_cap = batch, n_kv_heads, head_dim, t_cap
        self.seg_len, self.dtype = seg_len, dtype
        self.n_q_heads, self.top_chunks, self.top_groups = n_q_heads, top_chunks, top_groups
        self.k_host = torch.zeros(batch, n_kv_heads, t_cap, head_dim, dtype=dtype, pin_memory=True)
        self.v_host = torch.zeros_like(self.k_host, pin_memory=True)
        self.gsum = torch.zeros(batch, n_kv_heads, t_cap // 8, head_dim, dtype=dtype, device=device)
        self.csum = torch.zeros(batch, n_kv_heads, t_cap // 64, head_dim, dtype=dtype, device=device)
        shape = L.make_shape(batch, n_q_heads, n_kv_heads, head_dim, top_chunks, top_groups, _dtype_name(dtype))
        # one staging position for every segment: enough for any selection of the longest history
        self.stage_hist = max(64, L.hga_stage_history_min(shape, max(t_cap - seg_len, 0), seg_len))
        self.stage_cap = self.stage_hist + seg_len
        self.k_stage = torch.zeros(batch, n_kv_heads, self.stage_cap, head_dim, dtype=dtype, device=device)
        self.v_stage = torch.zeros_like(self.k_stage)
        self._gs_seg = torch.zeros(batch, n_kv_heads, self.stage_cap // 8, head_dim, dtype=dtype, device=device)
        self._cs_seg = torch.zeros(batch, n_kv_heads, self.stage_cap // 64, head_dim, dtype=dtype, device=device)
        self.length = 0
        self.q_last: Optional[torch.Tensor] = None      # [B, Hq, 64, d] of the committed history
        self._q_pending: Optional[torch.Tensor] = None
        self.k = self.k_stage        # the device tensor the segment's checks compare devices with

    def write(self, k_seg: torch.Tensor, v_seg: torch.Tensor, shape: L.HgaShape) -> int:
        """The active segment into the staging cache and its summaries into the
        tables (at its global position).  Returns the history length."""
        S = k_seg.shape[2]
        t0 = self.length
        if S != self.seg_len:
            raise ValueError(f"segments of this cache have {self.seg_len} tokens, got {S}")
        if t0 + S > self.t_cap:
            raise ValueError("KV cache capacity exceeded")
        sh = self.stage_hist
        self.k_stage[:, :, sh:sh + S].copy_(k_seg.detach())
        self.v_stage[:, :, sh:sh + S].copy_(v_seg.detach())
        L.hga_build_summaries(shape, self.k_stage, self.stage_cap, sh, sh + S, self._gs_seg, self._cs_seg)
        self.gsum[:, :, t0 // 8:(t0 + S) // 8].copy_(self._gs_seg[:, :, sh // 8:(sh + S) // 8])
        self.csum[:, :, t0 // 64:(t0 + S) // 64].copy_(self._cs_seg[:, :, sh // 64:(sh + S) // 64])
        return t0

    def stage(self, shape: L.HgaShape, t_hist: int, gidx: torch.Tensor) -> torch.Tensor:
        """The selected history groups into the staging cache; returns the selection
        renumbered for it."""
        gst = torch.empty_like(gidx)
        L.hga_stage_history(shape, self.k_host, self.v_host, self.t_cap, t_hist, self.seg_len, gidx, self.k_stage,
                            self.v_stage, self.stage_cap, self.stage_hist, gst)
        return gst

    def keep_last_query_block(self, q: torch.Tensor):
        """Remember the written segment's last 64 query rows (taken over by commit)."""
        self._q_pending = q[:, :, -64:].detach().contiguous().clone()

    def commit(self, seg_len: int):
        """The segment becomes history: its K/V go to host memory."""
        t0, sh = self.length, self.stage_hist
        self.k_host[:, :, t0:t0 + seg_len].copy_(self.k_stage[:, :, sh:sh + seg_len])
        self.v_host[:, :, t0:t0 + seg_len].copy_(self.v_stage[:, :, sh:sh + seg_len])
        self.length += seg_len
        self.q_last, self._q_pending = self._q_pending, None


def _check_segment(q: torch.Tensor, k_seg: torch.Tensor, v_seg: torch.Tensor, cache: "HGAKVCache"):
    """Host-side agreement of a segment's tensors with the cache they are attended
    against (dtype, head size, batch, KV heads, device): the library reads the
    cache with the dtype and head size of the call, so a mismatch would otherwise
    become out-of-bounds device accesses."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, Hq, S, d], got {tuple(q.shape)}")
    B, Hq, S, d = q.shape
    if q.dtype != cache.dtype:
        raise ValueError(f"q has dtype {q.dtype} but the cache holds {cache.dtype}")
    if d != cache.head_dim or B != cache.batch:
        raise ValueError(f"q [B={B}, d={d}] does not match the cache [B={cache.batch}, d={cache.head_dim}]")
    if Hq % cache.n_kv_heads != 0:
        raise ValueError(f"{Hq} query heads are not a multiple of the cache's {cache.n_kv_heads} KV heads")
    if S <= 0 or S % 64 != 0:
        raise ValueError(f"segment length {S} must be a positive multiple of 64")
    want = (B, cache.n_kv_heads, S, d)
    for name, t in (("k_seg", k_seg), ("v_seg", v_seg)):
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must be {list(want)}, got {list(t.shape)}")
        if t.dtype != cache.dtype:
            raise ValueError(f"{name} has dtype {t.dtype} but the cache holds {cache.dtype}")
    for name, t in (("q", q), ("k_seg", k_seg), ("v_seg", v_seg)):
        if t.device != cache.k.device:
            raise ValueError(f"{name} is on {t.device}, the cache on {cache.k.device}")


class _HGAAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k_seg, v_seg, cache: HGAKVCache, top_chunks: int, top_groups: int, scale: float,
                causal_routing: bool):
        _check_segment(q, k_seg, v_seg, cache)
        B, Hq, S, d = q.shape
        shape = L.make_shape(B, Hq, cache.n_kv_heads, d, top_chunks, top_groups, _dtype_name(q.dtype), scale)
        q = q.contiguous()
        if causal_routing and cache.length > 0 and (cache.q_last is None or cache.q_last.shape[1] != Hq):
            raise ValueError("causal routing over history needs the previous segment's last query block "
                             "(route every segment of the cache causally)")
        nb = S // 64
        cidx = torch.empty(B, cache.n_kv_heads, nb, top_chunks, dtype=torch.int32, device=q.device)
        gidx = torch.empty(B, cache.n_kv_heads, nb, top_groups, dtype=torch.int32, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
        if isinstance(cache, HGAHostKVCache):
            # host-RAM tier: route over the tables in HBM (block j by its own rows, or
            # strictly causally by block j-1's), stage the selected history groups,
            # attend on the staging cache
            if Hq != cache.n_q_heads or top_groups > cache.top_groups:
                raise ValueError(f"this host-tier cache was sized for {cache.n_q_heads} query heads and at most "
                                 f"{cache.top_groups} groups per block, got {Hq} and {top_groups}")
            t_hist = cache.write(k_seg, v_seg, shape)
            if causal_routing:
                L.hga_route_causal(shape, q, cache.q_last if t_hist > 0 else None, cache.csum, cache.gsum,
                                   cache.t_cap, t_hist, S, cidx, gidx)
            else:
                L.hga_route(shape, q, cache.csum, cache.gsum, cache.t_cap, t_hist, S, cidx, gidx)
            gst = cache.stage(shape, t_hist, gidx)
            L.hga_attend_fwd(shape, q, cache.k_stage, cache.v_stage, cache.stage_cap, cache.stage_hist, S, gst, o,
                             lse)
            ctx.save_for_backward(q, o, lse, gst)
            ctx.cache, ctx.shape = cache, shape
            ctx.kv = (cache.k_stage, cache.v_stage, cache.stage_cap, cache.stage_hist)
            ctx.mark_non_differentiable(lse, gidx)
            cache.keep_last_query_block(q)
            return o, lse, gidx
        if causal_routing:
            # summaries of the segment, causal routing and attention in one call
            t_hist = cache.write(k_seg, v_seg, shape, summaries=False)
            L.hga_forward_causal(shape, q, cache.q_last if t_hist > 0 else None, cache.k, cache.v, cache.csum,
                                 cache.gsum, cache.t_cap, t_hist, S, cidx, gidx, o, lse)
        else:
            # summaries of the segment, routing and attention in one call
            t_hist = cache.write(k_seg, v_seg, shape, summaries=False)
            L.hga_forward(shape, q, cache.k, cache.v, cache.csum, cache.gsum, cache.t_cap, t_hist, S, cidx, gidx,
                          o, lse)
        cache.keep_last_query_block(q)
        ctx.save_for_backward(q, o, lse, gidx)
        ctx.cache, ctx.shape = cache, shape
        ctx.kv = (cache.k, cache.v, cache.t_cap, t_hist)
        ctx.mark_non_differentiable(lse, gidx)
        return o, lse, gidx

    @staticmethod
    def backward(ctx, d_o, _lse, _g):
        q, o, lse, gidx = ctx.saved_tensors
        cache, shape = ctx.cache, ctx.shape
        k, v, t_cap, t_hist = ctx.kv
        B, Hq, S, d = q.shape
        dq = torch.empty_like(q)
        dk = torch.empty(B, cache.n_kv_heads, S, d, dtype=q.dtype, device=q.device)
        dv = torch.empty_like(dk)
        ws = torch.empty(max(L.hga_attend_bwd_workspace_size(shape, t_hist, S), L.HGA_BWD_WORKSPACE_CLEAR_BYTES),
                         dtype=torch.uint8, device=q.device)
        ws[:L.HGA_BWD_WORKSPACE_CLEAR_BYTES].zero_()
        L.hga_attend_bwd(shape, q, k, v, o, lse, d_o.contiguous(), t_cap, t_hist, S, gidx, dq, dk, dv, ws)
        return dq, dk, dv, None, None, None, None, None


def hga_attention(q: torch.Tensor, k_seg: torch.Tensor, v_seg: torch.Tensor, cache: HGAKVCache,
                  top_chunks: int = 16, top_groups: int = 64, softmax_scale: Optional[float] = None,
                  causal_routing: bool = False):
    """Routed attention of one active segment against the cache's history plus itself.

    q [B,Hq,S,d], k_seg/v_seg [B,Hkv,S,d] (the segment's keys/values, written into
    the cache at its current length; same dtype, batch, KV heads and head size as
    the cache).  Returns (o [B,Hq,S,d], lse [B,Hq,S] float32, group_idx); lse and
    group_idx carry no gradient.  Call
    cache.commit(S) once the segment's backward is done to turn it into history.
    causal_routing: route each block with the block before it (hga_route_causal);
    then every segment written to the cache must be routed that way.
    """
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    return _HGAAttentionFn.apply(q, k_seg, v_seg, cache, top_chunks, top_groups, scale, causal_routing)


class HGAStack:
    """Segment-wise truncated backpropagation through a stack of HGA attention
    layers, the pages' training scheme (adnankhan.ai note, "Raw Abstract /
    Excerpt": only the active segment is differentiable, older K/V detached;
    seventnews, "HGA的不同之处": 2,048-token segments, each with its own forward
    and backward).  Every layer has its own K/V cache with summary tables.

    layers[l] supplies the model around the attention of layer l:
        qkv(h) -> (q [B,Hq,S,d], k [B,Hkv,S,d], v [B,Hkv,S,d])   differentiable
        out(h, o) -> h_next                                       differentiable
    run_segment(h, loss_fn) runs one segment: for each layer, qkv, routed attention
    over that layer's cache (history) and the segment itself, out; then
    loss_fn(h_last).backward(); then every cache commits the segment, whose K/V
    become detached history for the next segment (no gradient ever reaches them).
    budgets: one (top_chunks, top_groups) pair for every layer, or a list of them.
    host_history: keep every layer's detached history in pinned host memory
    (HGAHostKVCache; needs seg_len, the fixed segment length, and n_q_heads);
    results are bit-identical to the all-HBM caches.
    """

    def __init__(self, layers, batch: int, n_kv_heads: int, head_dim: int, t_cap: int, budgets=(16, 64),
                 dtype: torch.dtype = torch.bfloat16, device="cuda", softmax_scale: Optional[float] = None,
                 causal_routing: bool = False, host_history: bool = False, seg_len: Optional[int] = None,
                 n_q_heads: Optional[int] = None):
        self.layers = list(layers)
        n = len(self.layers)
        if isinstance(budgets[0], (tuple, list)):
            if len(budgets) != n:
                raise ValueError(f"{len(budgets)} budgets for {n} layers")
            self.budgets = [tuple(b) for b in budgets]
        else:
            self.budgets = [tuple(budgets)] * n
        if host_history:
            if seg_len is None or n_q_heads is None:
                raise ValueError("a host-memory history needs seg_len and n_q_heads (they size its staging cache)")
            self.caches = [HGAHostKVCache(batch, n_kv_heads, head_dim, t_cap, seg_len, n_q_heads, kc, kg, dtype,
                                          device) for kc, kg in self.budgets]
        else:
            self.caches = [HGAKVCache(batch, n_kv_heads, head_dim, t_cap, dtype, device) for _ in range(n)]
        self.softmax_scale = softmax_scale
        self.causal_routing = causal_routing
        self.segments = 0

    @property
    def length(self) -> int:
        """Tokens already committed as history."""
        return self.caches[0].length if self.caches else 0

    def run_segment(self, h, loss_fn):
        """Forward, backward and detach of one segment.  Returns (loss value, and per
        layer (o, lse, group_idx) of the segment, detached)."""
        outs = []
        seg_len = None
        for layer, cache, (kc, kg) in zip(self.layers, self.caches, self.budgets):
            q, k, v = layer.qkv(h)
            if seg_len is None:
                seg_len = q.shape[2]
            elif q.shape[2] != seg_len:
                raise ValueError("every layer must see the same segment length")
            o, lse, gidx = hga_attention(q, k, v, cache, kc, kg, self.softmax_scale, self.causal_routing)
            outs.append((o.detach(), lse, gidx))
            h = layer.out(h, o)
        loss = loss_fn(h)
        loss.backward()
        for cache in self.caches:
            cache.commit(seg_len)
        self.segments += 1
        return loss.detach(), outs


class HGADecoder:
    """Generation steps over `cache`: every sequence adds one token per step.

    step(q, k_new, v_new, pos) writes the new tokens' K/V at positions pos (a [B]
    int32 device tensor; an entry outside [0, t_cap) marks an idle slot, whose
    outputs are O = 0, LSE = -inf and no selection), routes each token
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
        B, Hq, Hkv, d = self.shape.batch, self.shape.n_q_heads, c.n_kv_heads, c.head_dim
        if tuple(q.shape) != (B, Hq, d) or q.dtype != c.dtype or q.device != c.k.device:
            raise ValueError(f"q must be [{B}, {Hq}, {d}] {c.dtype} on {c.k.device}, got "
                             f"{list(q.shape)} {q.dtype} on {q.device}")
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if tuple(t.shape) != (B, Hkv, d):
                raise ValueError(f"{name} must be [{B}, {Hkv}, {d}], got {list(t.shape)}")
        if tuple(pos.shape) != (B,) or pos.dtype != torch.int32 or pos.device != c.k.device:
            raise ValueError(f"pos must be a [{B}] int32 tensor on {c.k.device}")
        live = (pos >= 0) & (pos < c.t_cap)      # the library treats the other slots as idle
        bi, p = self._b[live], pos[live].long()
        c.k[bi, :, p] = k_new[live].to(c.dtype)
        c.v[bi, :, p] = v_new[live].to(c.dtype)
        L.hga_decode_step(self.shape, q.contiguous(), c.k, c.v, c.csum, c.gsum, c.t_cap, pos, self.cidx,
                          self.gidx, self.o, self.lse, self.ws)
        return self.o, self.lse, self.gidx
