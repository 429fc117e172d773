// Two-level routing of one (sequence, KV head, query block) unit on the matrix
// cores: chunk scores -> top-k chunks -> group scores -> top-k groups.  Shared by
// the routing kernel (route.hip) and by the forward kernel that routes and then
// attends in one work-group (attend_fwd.hip).
//
// Pages: seventnews "BMW如何通过重新设计注意力机制，在16 GB GPU上实现16K上下文", section
// "HGA的不同之处" (queries score the chunk summaries, keep the top-k chunks, open
// them at group level; no learned router weights) and section "一个真正的警告：
// 因果泄露" (one decision per block from the scores of several query positions).
// Readings of this library: the per-row score is q . summary in fp32; the block
// score is the maximum over the block's rows (64 positions x the query heads of
// the KV head); candidates are every complete chunk before the block; groups are
// the 8 groups of every selected chunk; ties go to the lower index; outputs are
// ascending and padded with -1.  Strictly causal variant: a block is routed by the
// rows of the query block before it (RouteArgs::lag).
//
// Scoring uses v_mfma_f32_32x32x16_bf16 with operand A = 32 query rows (held in
// registers) and operand B = 32 summary rows staged in swizzled LDS tiles, so each
// lane ends with one candidate column and 16 of the rows and the row maximum is a
// register reduction plus one cross-half exchange.  Block maxima of the waves meet
// in LDS through an atomic max on order-preserving integer keys.  The top-k (up to
// 512 candidates) is one wave's most-significant-bit-first search for the k-th
// largest (key, index) pair, counting with ballots, then an index-ordered
// compaction; above 512 candidate chunks every wave keeps the best k_c of its share
// and one wave selects among those.  All exact and deterministic, ties by index.
#pragma once

#include "hga_device.h"
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

// Rows of the block: row = hh * 64 + pos (hh = query head within the KV group).
// Row tile rt (32 rows) belongs to waves rt % 4 (and rt % 4 + 4).  Candidate
// summaries are copied into swizzled LDS tiles in batches of 128 rows (two
// buffers: the next batch is copied while one is scored) and scored from there:
// each batch is read from memory once per work-group.
constexpr int kBatch = 128;   // summary rows per batch (two 64-row tiles)

// Threads of the bf16 router: 8 waves, two per SIMD, up to 4 query heads per KV head;
// with 8 heads the row tiles take the registers of a wave per SIMD.
template <int G>
constexpr int route_threads() { return G >= 8 ? 256 : kRouteThreads; }
template <int G>
constexpr int route_row_tiles_per_wave() { return (2 * G + 3) / 4; }

template <int NT>
struct RouteShared {
  uint32_t ckeys[kMaxChunks + 4];
  uint32_t gkeys[kMaxGroupCand + 4];
  int csel[64];
  int gsel[kMaxGroupCand];
  TopkShared<NT> top;
  int nsel;
};

// Selection of unit `unit` (all threads of the work-group call it).  tile(B, T)
// gives the LDS address of 64-row half T of summary batch buffer B (B, T in {0, 1},
// as ic<> constants; kBatch x D bf16 per buffer).  On return qf holds the routing
// rows (lane row n of row tiles wr, wr + 4, ...; zero for tiles past the block or
// when nothing is scored), sm.csel[0 .. nc) the chosen chunks ascending and
// sm.gsel[0 .. ng) the chosen group slots ascending (slot s = group 8 csel[s/8] +
// s%8, so ascending slots are ascending ids); chunk_idx / group_idx (and the
// optional scores) of the unit are written.  The selections are visible to every
// thread on return, and no wave reads the batch buffers any more.  after_chunks()
// runs in every thread once the chunk scores are complete (before the selection):
// a caller may issue its own asynchronous copies there.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};
template <int D, int G, typename Tile, typename AfterChunks = NoHook>
__device__ __forceinline__ void route_unit_bf16(const RouteArgs& a, int unit, const Tile& tile,
                                                RouteShared<route_threads<G>()>& sm,
                                                bf16x8 (&qf)[route_row_tiles_per_wave<G>()][D / 16], int& nc_out,
                                                int& ng_out, const AfterChunks& after_chunks = AfterChunks{}) {
  constexpr int NT = route_threads<G>();
  constexpr int KS = D / 16;
  constexpr int NRT = 2 * G;                      // 32-row tiles in the block
  constexpr int RPW = route_row_tiles_per_wave<G>();
  constexpr int NW = NT / 64;
  constexpr int SPW = 8 / NW;                     // pairs of a batch's 32-row subtiles per wave
  uint32_t* ckeys = sm.ckeys;
  uint32_t* gkeys = sm.gkeys;
  int* csel = sm.csel;
  int* gsel = sm.gsel;

  const int j = unit % a.nb;
  const int bh = unit / a.nb;                     // b * Hkv + kvh
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x, w = tid >> 6, h = (tid & 63) >> 5, n = tid & 31;
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
      dma_tile<D, NW>(tile(B, T), [&](int r) { return row_src(min(r0 + 64 * T() + r, n_rows - 1)); });
    });
  };
  // Batch 0 must already be in flight (issue_rows(n_rows, row_src, 0, ic<0>)).
  auto score_rows = [&](int n_rows, auto&& row_src, uint32_t* keys) __attribute__((always_inline)) {
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
          // With 8 waves, waves w and w + 4 hold the same row tiles and score one pair of
          // the batch's four 32-row subtiles each (two waves per SIMD); with 4 waves a
          // wave scores both pairs in turn.  Two independent MFMA chains per row tile.
          static_for<0, 2>([&](auto SP) {
            const int sp = SP();
            if (sp >= sp0 && sp < sp0 + SPW) {
              const uint16_t* tb = tile(B, SP);
              bf16x8 bfr[2][KS];
              static_for<0, 2>([&](auto U) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) bfr[U()][ks] = ro.template read<U() * 32 * D * 2>(tb, ks);
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
          });
        }
      });
    }
  };

  auto chunk_row = [&](int r) __attribute__((always_inline)) { return cs + (int64_t)r * D; };
  if (J > 0) issue_rows(J, chunk_row, 0, ic<0>{});   // the first summaries travel while Q loads

  // Query fragments (MFMA operand A): lane holds row n of each of its row tiles.
  // Nothing is scored when J == 0; the rows are still loaded then under block
  // routing (a caller may attend with them), but not under causal routing (q_prev
  // may be absent).
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int rt = wr + 4 * i;
    if (rt < NRT && (J > 0 || a.lag == 0)) {
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
  if (J > 0) score_rows(J, chunk_row, ckeys);
  __syncthreads();
  after_chunks();
  // ascending chunk ids: one wave's bit search up to 512 candidates; above, every
  // wave keeps the best k_c of its share and one wave selects among those
  const int nc = (J == 0 || a.kc == 0) ? 0
                 : J <= 64              ? wave_topk_sorted<1>(ckeys, J, a.kc, csel, &sm.nsel)
                 : J <= 128             ? wave_topk_sorted<2>(ckeys, J, a.kc, csel, &sm.nsel)
                 : J <= 256             ? wave_topk_sorted<4>(ckeys, J, a.kc, csel, &sm.nsel)
                 : J <= 512             ? wave_topk_sorted<8>(ckeys, J, a.kc, csel, &sm.nsel)
                                        : topk64(sm.top, J, a.kc, csel, (uint32_t*)nullptr,
                                                 [&](int i) { return cand(ckeys[i], i); });

  // ---- group scores over the 8 groups of each selected chunk, then top-k_g
  const int ng_cand = 8 * nc;
  for (int i = tid; i < ((ng_cand + 3) & ~3); i += NT) gkeys[i] = 0u;
  __syncthreads();
  if (ng_cand > 0) {
    auto group_row = [&](int r) __attribute__((always_inline)) { return gs + (int64_t)(8 * csel[r >> 3] + (r & 7)) * D; };
    issue_rows(ng_cand, group_row, 0, ic<0>{});
    score_rows(ng_cand, group_row, gkeys);
  }
  __syncthreads();
  const int ng = (ng_cand == 0 || a.kg == 0) ? 0        // ascending slots == ascending ids
                 : ng_cand <= 64  ? wave_topk_sorted<1>(gkeys, ng_cand, a.kg, gsel, &sm.nsel)
                 : ng_cand <= 128 ? wave_topk_sorted<2>(gkeys, ng_cand, a.kg, gsel, &sm.nsel)
                 : ng_cand <= 256 ? wave_topk_sorted<4>(gkeys, ng_cand, a.kg, gsel, &sm.nsel)
                                  : wave_topk_sorted<8>(gkeys, ng_cand, a.kg, gsel, &sm.nsel);

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
  nc_out = nc;
  ng_out = ng;
}

}  // namespace
}  // namespace hga
