// Two-level routing: chunk scores -> top-k chunks -> group scores -> top-k groups.
//
// Pages: seventnews "BMW如何通过重新设计注意力机制，在16 GB GPU上实现16K上下文", section
// "HGA的不同之处" (queries score the chunk summaries, keep the top-k chunks, open
// them at group level; no learned router weights) and section "一个真正的警告：
// 因果泄露" (one decision per block from the scores of several query positions).
// Readings of this library: the per-row score is q . summary in fp32; the block
// score is the maximum over the block's rows (64 positions x the query heads of
// the KV head); candidates are every complete chunk before the block; groups are
// the 8 groups of every selected chunk; ties go to the lower index; outputs are
// ascending and padded with -1.
//
// Strictly causal variant (the same article, "因果泄露", says one is in development
// and gives no design; this library's reading): a block is routed by the rows of
// the query block before it -- block j-1 of the segment, or for j = 0 the last
// block of the previous segment (q_prev) -- with the same candidates, so no input
// of the decision lies at or after the block's first position.  Only the source
// of the query rows differs (RouteArgs::lag).
//
// One work-group per (sequence, KV head, query block).  The bf16
// path scores with v_mfma_f32_32x32x16_bf16: operand A = 32 query rows (held in
// registers for the whole kernel), operand B = 32 summary rows, so each lane
// ends with one candidate column and 16 of the rows and the row-maximum is a
// register reduction plus one cross-half exchange.  Block maxima of the waves
// meet in LDS through an atomic max on order-preserving integer keys.  The top-k
// (up to 512 candidates) is one wave's most-significant-bit-first search for the
// k-th largest (key, index) pair, counting with ballots, then an index-ordered
// compaction; above 512 candidate chunks every wave keeps the best k_c of its
// share the same way and one wave selects among those.  All are exact and
// deterministic, ties resolved by index.  The fp32 path uses a block-wide radix
// select.
#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"

#include <math.h>

namespace hga {
namespace {


struct RouteArgs {
  const void* q;
  const void* q_prev;   // [B, Hq, 64, d]: routes block 0 when lag == 1
  const void* csum;
  const void* gsum;
  int32_t* cidx;
  int32_t* gidx;
  float* cscore;
  float* gscore;
  int64_t t_cap, t_hist, seg_len;
  int Hq, Hkv, kc, kg, nb, n_units;
  int lag;              // 0: a block routes itself; 1: the block before it routes it
};

// Start of query row `pos` of head `head` in the block that routes block j.
template <typename T>
__device__ __forceinline__ const T* routing_row(const RouteArgs& a, int b, int head, int j, int pos, int D) {
  const int qb = j - a.lag;
  if (qb >= 0)
    return (const T*)a.q + ((((int64_t)b * a.Hq + head) * a.seg_len) + qb * kQBlock + pos) * D;
  return (const T*)a.q_prev + ((((int64_t)b * a.Hq + head) * kQBlock) + pos) * D;
}

// ---------------------------------------------------------------- bf16 / MFMA
// Rows of the block: row = hh * 64 + pos (hh = query head within the KV group).
// Row tile rt (32 rows) belongs to waves rt % 4 (and rt % 4 + 4).  Candidate summaries are copied
// into swizzled LDS tiles in batches of 128 rows (two buffers: the next batch
// is copied while one is scored) and scored from there: each batch is read from
// memory once per work-group.
constexpr int kBatch = 128;   // summary rows per batch (two 64-row tiles)

// Threads of the bf16 router: 8 waves, two per SIMD, up to 4 query heads per KV head;
// with 8 heads the row tiles take the registers of a wave per SIMD.
template <int G>
constexpr int route_threads() { return G >= 8 ? 256 : kRouteThreads; }

template <int D, int G>
__global__ __launch_bounds__(route_threads<G>()) void route_bf16_kernel(RouteArgs a) {
  constexpr int NT = route_threads<G>();
  constexpr int KS = D / 16;
  constexpr int NRT = 2 * G;                      // 32-row tiles in the block
  constexpr int RPW = (NRT + 3) / 4;              // row tiles per wave
  constexpr int NW = NT / 64;
  constexpr int SPW = 8 / NW;                     // pairs of a batch's 32-row subtiles per wave
  constexpr int L = 2 * dma_per_wave<D, NW>();    // copies per wave per batch
  __shared__ __align__(16) uint16_t sb0[kBatch * D], sb1[kBatch * D];
  __shared__ __align__(16) uint32_t ckeys[kMaxChunks + 4];
  __shared__ __align__(16) uint32_t gkeys[kMaxGroupCand + 4];
  __shared__ int csel[64];
  __shared__ int gsel[kMaxGroupCand];
  __shared__ TopkShared<NT> top;
  __shared__ int nsel;
  auto SB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return sb0; else return sb1;
  };

  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int j = unit % a.nb;
  const int bh = unit / a.nb;                     // b * Hkv + kvh
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = l & 31;
  const int wr = w & 3, sp0 = (w >> 2) * SPW;   // row-tile set; first subtile pair of a batch

  const uint16_t* cs = (const uint16_t*)a.csum + (int64_t)bh * (a.t_cap / kChunk) * D;
  const uint16_t* gs = (const uint16_t*)a.gsum + (int64_t)bh * (a.t_cap / kGroup) * D;

  // Score rows [0, n_rows) given row_src(r) (global address of summary row r, r < n_rows):
  // the block maximum of q . row goes to keys[r] as an orderable key.
  RowOffsets<D> ro;
  ro.init(n, h);
  // Copies of batch bt of rows [0, n_rows) into buffer set B.
  auto issue_rows = [&](int n_rows, auto&& row_src, int bt, auto B) __attribute__((always_inline)) {
    const int r0 = bt * kBatch;
    static_for<0, 2>([&](auto T) {
      dma_tile<D, NW>(SB(B) + T() * 64 * D, [&](int r) { return row_src(min(r0 + 64 * T() + r, n_rows - 1)); });
    });
  };
  // Batch 0 must already be in flight (issue_rows(n_rows, row_src, 0, ic<0>)).
  auto score_rows = [&](int n_rows, auto&& row_src, uint32_t* keys, const bf16x8 (&qf)[RPW][KS]) __attribute__((always_inline)) {
    auto issue = [&](int bt, auto B) __attribute__((always_inline)) { issue_rows(n_rows, row_src, bt, B); };
    const int n_batches = (n_rows + kBatch - 1) / kBatch;
    for (int bt0 = 0; bt0 < n_batches; bt0 += 2) {
      static_for<0, 2>([&](auto B) {
        const int bt = bt0 + B();
        if (bt < n_batches) {
          wait_vmcnt<0>();
          tile_barrier();   // batch bt visible; every wave is done with batch bt-1's buffer
          if (bt + 1 < n_batches) issue(bt + 1, ic<1 - B()>{});
          ro.refresh();
          const uint16_t* tb = SB(B);
          // With 8 waves, waves w and w + 4 hold the same row tiles and score one pair of
          // the batch's four 32-row subtiles each (two waves per SIMD); with 4 waves a
          // wave scores both pairs in turn.  Two independent MFMA chains per row tile.
          for (int sp = sp0; sp < sp0 + SPW; ++sp) {
            bf16x8 bfr[2][KS];
            static_for<0, 2>([&](auto U) {
#pragma unroll
              for (int ks = 0; ks < KS; ++ks)
                bfr[U()][ks] = ro.template read<U() * 32 * D * 2>(tb + sp * 64 * D, ks);
            });
            float best[2] = {-INFINITY, -INFINITY};
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              if (NRT % 4 == 0 || wr + 4 * i < NRT) {
                f32x16 acc[2] = {};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                  for (int u = 0; u < 2; ++u) acc[u] = mfma32(qf[i][ks], bfr[u][ks], acc[u]);
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                  for (int rr = 0; rr < 16; ++rr) best[u] = fmaxf(best[u], acc[u][rr]);
              }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = bt * kBatch + 64 * sp + 32 * u + n;
              const float bb = half_max(best[u]);
              if (h == 0 && r < n_rows && wr < NRT) atomicMax(&keys[r], score_key(bb));
            }
          }
        }
      });
    }
  };

  auto chunk_row = [&](int r) __attribute__((always_inline)) { return cs + (int64_t)r * D; };
  if (J > 0) issue_rows(J, chunk_row, 0, ic<0>{});   // the first summaries travel while Q loads

  // Query fragments (MFMA operand A): lane holds row n of each of its row tiles.
  // Nothing is scored when J == 0 (and q_prev may then be absent).
  bf16x8 qf[RPW][KS];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int rt = wr + 4 * i;
    if (rt < NRT && J > 0) {
      const int hh = rt >> 1, pos = 32 * (rt & 1) + n;
      const uint16_t* qp = routing_row<uint16_t>(a, b, kvh * G + hh, j, pos, D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[i][ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[i][ks] = bf16x8{};
    }
  }

  // ---- chunk scores and top-k_c over the candidate chunks [0, J)
  for (int i = tid; i < ((J + 3) & ~3); i += NT) ckeys[i] = 0u;
  __syncthreads();
  if (J > 0) score_rows(J, chunk_row, ckeys, qf);
  __syncthreads();
  // ascending chunk ids: one wave's bit search up to 512 candidates; above, every
  // wave keeps the best k_c of its share and one wave selects among those
  const int nc = (J == 0 || a.kc == 0) ? 0
                 : J <= 64              ? wave_topk_sorted<1>(ckeys, J, a.kc, csel, &nsel)
                 : J <= 128             ? wave_topk_sorted<2>(ckeys, J, a.kc, csel, &nsel)
                 : J <= 256             ? wave_topk_sorted<4>(ckeys, J, a.kc, csel, &nsel)
                 : J <= 512             ? wave_topk_sorted<8>(ckeys, J, a.kc, csel, &nsel)
                                        : topk64(top, J, a.kc, csel, (uint32_t*)nullptr,
                                                 [&](int i) { return cand(ckeys[i], i); });

  // ---- group scores over the 8 groups of each selected chunk, then top-k_g
  const int ng_cand = 8 * nc;
  for (int i = tid; i < ((ng_cand + 3) & ~3); i += NT) gkeys[i] = 0u;
  __syncthreads();
  if (ng_cand > 0) {
    auto group_row = [&](int r) __attribute__((always_inline)) { return gs + (int64_t)(8 * csel[r >> 3] + (r & 7)) * D; };
    issue_rows(ng_cand, group_row, 0, ic<0>{});
    score_rows(ng_cand, group_row, gkeys, qf);
  }
  __syncthreads();
  const int ng = (ng_cand == 0 || a.kg == 0) ? 0        // ascending slots == ascending ids
                 : ng_cand <= 64  ? wave_topk_sorted<1>(gkeys, ng_cand, a.kg, gsel, &nsel)
                 : ng_cand <= 128 ? wave_topk_sorted<2>(gkeys, ng_cand, a.kg, gsel, &nsel)
                 : ng_cand <= 256 ? wave_topk_sorted<4>(gkeys, ng_cand, a.kg, gsel, &nsel)
                                  : wave_topk_sorted<8>(gkeys, ng_cand, a.kg, gsel, &nsel);

  // ---- outputs
  int32_t* co = a.cidx + (int64_t)unit * a.kc;
  int32_t* go = a.gidx + (int64_t)unit * a.kg;
  for (int i = tid; i < a.kc; i += NT) {
    co[i] = i < nc ? csel[i] : -1;
    if (a.cscore) a.cscore[(int64_t)unit * a.kc + i] = i < nc ? key_score(ckeys[csel[i]]) : -INFINITY;
  }
  for (int i = tid; i < a.kg; i += NT) {
    const int slot = i < ng ? gsel[i] : 0;
    go[i] = i < ng ? 8 * csel[slot >> 3] + (slot & 7) : -1;
    if (a.gscore) a.gscore[(int64_t)unit * a.kg + i] = i < ng ? key_score(gkeys[slot]) : -INFINITY;
  }
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
hipError_t launch_bf16(const RouteArgs& a, int grid, hipStream_t s) {
  return launch_kernel(route_bf16_kernel<D, G>, dim3(grid), dim3(route_threads<G>()), s, a);
}

template <int D>
hipError_t launch_bf16_g(const RouteArgs& a, int G, int grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_bf16<D, 1>(a, grid, s);
    case 2: return launch_bf16<D, 2>(a, grid, s);
    case 4: return launch_bf16<D, 4>(a, grid, s);
    default: return launch_bf16<D, 8>(a, grid, s);
  }
}

}  // namespace

hipError_t launch_route(const Dims& d, bool bf16, const void* q, const void* q_prev, bool causal,
                        const void* chunk_sum, const void* group_sum, int32_t* chunk_idx,
                        int32_t* group_idx, float* chunk_score, float* group_score, hipStream_t s) {
  RouteArgs a;
  a.q = q; a.q_prev = q_prev; a.lag = causal ? 1 : 0;
  a.csum = chunk_sum; a.gsum = group_sum;
  a.cidx = chunk_idx; a.gidx = group_idx; a.cscore = chunk_score; a.gscore = group_score;
  a.t_cap = d.t_cap; a.t_hist = d.t_hist; a.seg_len = d.seg_len;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kc = d.kc; a.kg = d.kg; a.nb = d.nb;
  a.n_units = d.B * d.Hkv * d.nb;
  const int grid = xcd_grid(a.n_units);
  if (bf16) return d.D == 128 ? launch_bf16_g<128>(a, d.G, grid, s) : launch_bf16_g<64>(a, d.G, grid, s);
  return d.D == 128 ? launch_kernel(route_f32_kernel<128>, dim3(grid), dim3(kRouteThreadsF32), s, a, d.G)
                    : launch_kernel(route_f32_kernel<64>, dim3(grid), dim3(kRouteThreadsF32), s, a, d.G);
}

}  // namespace hga
