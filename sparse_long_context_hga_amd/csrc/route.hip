// Two-level routing: chunk scores -> top-k chunks -> group scores -> top-k groups,
// one work-group per (sequence, KV head, query block).  The bf16 path is the
// matrix-core selection of route_phase.h (also used by the forward kernel that
// routes and attends in one work-group); the fp32 path scores on the vector ALUs
// and selects with a block-wide radix select.
//
// Pages: seventnews "BMW如何通过重新设计注意力机制，在16 GB GPU上实现16K上下文", section
// "HGA的不同之处" (queries score the chunk summaries, keep the top-k chunks, open
// them at group level; no learned router weights) and section "一个真正的警告：
// 因果泄露" (one decision per block from the scores of several query positions).
//
// Strictly causal variant (the same article, "因果泄露", says one is in development
// and gives no design; this library's reading): a block is routed by the rows of
// the query block before it -- block j-1 of the segment, or for j = 0 the last
// block of the previous segment (q_prev) -- with the same candidates, so no input
// of the decision lies at or after the block's first position.  Only the source
// of the query rows differs (RouteArgs::lag).
#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"
#include "route_phase.h"

#include <math.h>

namespace hga {
namespace {

// ---------------------------------------------------------------- bf16 / MFMA
template <int D, int G>
__global__ __launch_bounds__(route_threads<G>()) void route_bf16_kernel(RouteArgs a) {
  __shared__ __align__(16) uint16_t sb0[kBatch * D], sb1[kBatch * D];
  __shared__ RouteShared<route_threads<G>()> sm;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  auto tile = [&](auto B, auto T) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return sb0 + T() * 64 * D; else return sb1 + T() * 64 * D;
  };
  bf16x8 qf[route_row_tiles_per_wave<G>()][D / 16];
  int nc, ng;
  route_unit_bf16<D, G>(a, unit, tile, sm, qf, nc, ng);
}

// ---------------------------------------------------------------- fp32 (SIMT)
// Same routing with fp32 dot products on the vector ALUs (exact-precision mode).
template <int D>
__global__ __launch_bounds__(kRouteThreadsF32) void route_f32_kernel(RouteArgs a, int G) {
  __shared__ uint32_t ckeys[kMaxChunks];
  __shared__ uint32_t gkeys[kMaxGroupCand];
  __shared__ int csel[64];
  __shared__ int gsel[kMaxGroupCand];
  __shared__ SelectShared<kRouteThreadsF32> sh;

  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int j = unit % a.nb;
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x;
  const float* cs = (const float*)a.csum + (int64_t)bh * (a.t_cap / kChunk) * D;
  const float* gs = (const float*)a.gsum + (int64_t)bh * (a.t_cap / kGroup) * D;
  const int R = G * kQBlock;

  auto block_max = [&](const float* srow) {
    float best = -INFINITY;
    for (int r = 0; r < R; ++r) {
      const int hh = r / kQBlock, pos = r % kQBlock;
      const float* qp = routing_row<float>(a, b, kvh * G + hh, j, pos, D);
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc = fmaf(qp[e], srow[e], acc);
      best = fmaxf(best, acc);
    }
    return best;
  };

  for (int c = tid; c < J; c += kRouteThreadsF32) ckeys[c] = score_key(block_max(cs + (int64_t)c * D));
  __syncthreads();
  const int nc = block_topk(ckeys, J, a.kc, csel, sh);
  const int ng_cand = 8 * nc;
  for (int s = tid; s < ng_cand; s += kRouteThreadsF32)
    gkeys[s] = score_key(block_max(gs + (int64_t)(8 * csel[s >> 3] + (s & 7)) * D));
  __syncthreads();
  const int ng = block_topk(gkeys, ng_cand, a.kg, gsel, sh);

  int32_t* co = a.cidx + (int64_t)unit * a.kc;
  int32_t* go = a.gidx + (int64_t)unit * a.kg;
  for (int i = tid; i < a.kc; i += kRouteThreadsF32) {
    co[i] = i < nc ? csel[i] : -1;
    if (a.cscore) a.cscore[(int64_t)unit * a.kc + i] = i < nc ? key_score(ckeys[csel[i]]) : -INFINITY;
  }
  for (int i = tid; i < a.kg; i += kRouteThreadsF32) {
    const int slot = i < ng ? gsel[i] : 0;
    go[i] = i < ng ? 8 * csel[slot >> 3] + (slot & 7) : -1;
    if (a.gscore) a.gscore[(int64_t)unit * a.kg + i] = i < ng ? key_score(gkeys[slot]) : -INFINITY;
  }
}

template <int D, int G>
hipError_t launch_bf16(const RouteArgs& a, int grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  return launch_kernel_timed(route_bf16_kernel<D, G>, dim3(grid), dim3(route_threads<G>()), s, start, stop, a);
}

template <int D>
hipError_t launch_bf16_g(const RouteArgs& a, int G, int grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  switch (G) {
    case 1: return launch_bf16<D, 1>(a, grid, s, start, stop);
    case 2: return launch_bf16<D, 2>(a, grid, s, start, stop);
    case 4: return launch_bf16<D, 4>(a, grid, s, start, stop);
    default: return launch_bf16<D, 8>(a, grid, s, start, stop);
  }
}

}  // namespace

hipError_t launch_route(const Dims& d, bool bf16, const void* q, const void* q_prev, bool causal,
                        const void* chunk_sum, const void* group_sum, int32_t* chunk_idx,
                        int32_t* group_idx, float* chunk_score, float* group_score, hipStream_t s,
                        hipEvent_t start, hipEvent_t stop) {
  RouteArgs a;
  a.q = q; a.q_prev = q_prev; a.lag = causal ? 1 : 0;
  a.csum = chunk_sum; a.gsum = group_sum;
  a.cidx = chunk_idx; a.gidx = group_idx; a.cscore = chunk_score; a.gscore = group_score;
  a.t_cap = d.t_cap; a.t_hist = d.t_hist; a.seg_len = d.seg_len;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kc = d.kc; a.kg = d.kg; a.nb = d.nb;
  a.n_units = d.B * d.Hkv * d.nb;
  const int grid = xcd_grid(a.n_units);
  if (bf16)
    return d.D == 128 ? launch_bf16_g<128>(a, d.G, grid, s, start, stop) : launch_bf16_g<64>(a, d.G, grid, s, start, stop);
  return d.D == 128
             ? launch_kernel_timed(route_f32_kernel<128>, dim3(grid), dim3(kRouteThreadsF32), s, start, stop, a, d.G)
             : launch_kernel_timed(route_f32_kernel<64>, dim3(grid), dim3(kRouteThreadsF32), s, start, stop, a, d.G);
}

}  // namespace hga
