// Generation path: one new token per sequence, routed by its own query heads.
//
// Pages: the abstract on the adnankhan.ai note ("Raw Abstract / Excerpt") and the
// seventnews article (section "检索：密集基线无退化") say HGA can be used for
// generation and that a serving implementation is in development; they give no
// design.  This library's reading: the new token at position pos is a query
// block of one position, so the rows that score the summaries are its G query
// heads; the candidates are the chunks before its own (0 .. J-1, J = pos / 64);
// it attends the selected groups' exact tokens plus its own chunk up to and
// including itself.  Routing per token is strictly causal by construction.  When
// pos is the last position of a chunk, the chunk's group and chunk summaries are
// built (same fixed fp32 tree as hga_build_summaries) so later tokens can pick it.
//
// A step moves little data per (sequence, KV head) unit, and one compute unit
// alone cannot keep enough HBM requests in flight to move it quickly, so each
// unit is spread over many work-groups, and the last one to finish a phase
// finishes it (an arrival counter per unit, reset by that work-group):
//   route   work-group s scores candidate chunks 64s .. 64s+63 (16 lanes per
//           summary row, 16 B each); the last one selects the top-k_c chunks,
//           scores their groups and selects the top-k_g groups.
//   attend  work-group 0 takes the own chunk, work-group s >= 1 the selected
//           groups 8(s-1) .. 8s-1 (64 tokens, K and V rows read once); each
//           leaves a partial (max, sum, unnormalised O); the last one merges.
// Values that another work-group reads are written and read with device-scope
// (agent) coherent accesses, and a work-group's own stores complete before it
// arrives, so no cache-wide write-back or invalidation is needed.  Scores and
// attention are G-row GEMVs on the vector ALUs in fp32 (not GEMM-shaped, so no
// MFMA); selection uses ballot-counted bit searches on (score, index) keys.
#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"

#include <math.h>

namespace hga {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kSliceChunks = 64;   // candidate chunks scored per routing work-group
constexpr int kSplitGroups = 8;    // groups (64 tokens) per attention work-group

struct DecodeArgs {
  const void* q;          // [B, Hq, d]
  const void* k;          // [B, Hkv, t_cap, d]
  const void* v;
  const void* csum;       // [B, Hkv, t_cap/64, d]
  const void* gsum;       // [B, Hkv, t_cap/8, d]
  void* csum_out;         // summary tables updated by the attention (nullable)
  void* gsum_out;
  const int32_t* pos;     // [B]
  int32_t* cidx;          // [B, Hkv, k_c] (nullable)
  int32_t* gidx;          // [B, Hkv, k_g]
  const int32_t* gidx_in; // attention: the selection to attend
  float* cscore;
  float* gscore;
  void* o;                // [B, Hq, d]
  float* lse;             // [B, Hq]
  uint32_t* rcount;       // workspace: arrival counters [n_units]
  uint32_t* acount;       //            [n_units]
  uint64_t* cands;        //            best chunks of each slice [n_units][n_slices][k_c]
  float* part;            //            partials [n_units][n_split][G*(d+2)]
  int64_t t_cap;
  int Hq, Hkv, kc, kg, n_units, n_slices, n_split;
  float scale_log2;       // softmax_scale * log2(e)
};

// 8 consecutive elements of a row (16 B of bf16, 32 B of fp32), widened to fp32.
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  uint4 r = {0, 0, 0, 0};
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float* x) const {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Vec8<float> {
  float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* x) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

__device__ __forceinline__ void store_elem(uint16_t* p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void store_elem(float* p, float x) { *p = x; }
__device__ __forceinline__ float widen(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float widen(float x) { return x; }

__device__ __forceinline__ float tree8(const float* x) {
  const float a = (x[0] + x[1]) + (x[2] + x[3]);
  const float b = (x[4] + x[5]) + (x[6] + x[7]);
  return a + b;
}

// ------------------------------------------------ cross-lane reductions
// Within a row of 16 lanes through DPP (VALU, no LDS): quad_perm [1,0,3,2] and
// [2,3,0,1] pair the lanes of a quad, row_half_mirror pairs the two quads of each
// 8 lanes, row_mirror the two halves of the row.  Every pairing is symmetric, so
// all lanes of the group end with the same value.  Rows of a wave are then paired
// by an xor-16 swizzle and v_permlane32_swap.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t swz_xor16(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);   // and 0x1F, xor 0x10
}
__device__ __forceinline__ float fdpp_add(float x, uint32_t y) { return x + __uint_as_float(y); }

// Sum over the aligned groups of LPR lanes (8 or 16) that share a row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 8 || LPR == 16, "rows of 8 or 16 lanes");
  x = fdpp_add(x, dpp<0xB1>(__float_as_uint(x)));
  x = fdpp_add(x, dpp<0x4E>(__float_as_uint(x)));
  x = fdpp_add(x, dpp<0x141>(__float_as_uint(x)));
  if constexpr (LPR == 16) x = fdpp_add(x, dpp<0x140>(__float_as_uint(x)));
  return x;
}
// Sum over the lanes l, l + LPR, l + 2 LPR, ... of a wave (the rows of a column).
template <int LPR>
__device__ __forceinline__ float col_sum(float x) {
  if constexpr (LPR == 8) x = fdpp_add(x, dpp<0x128>(__float_as_uint(x)));   // row_ror 8: lane ^ 8
  x = fdpp_add(x, swz_xor16(__float_as_uint(x)));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_sum(float x) { return col_sum<16>(row_sum<16>(x)); }
__device__ __forceinline__ float wave_max(float x) {
  auto mx = [](float a, uint32_t b) { return fmaxf(a, __uint_as_float(b)); };
  x = mx(x, dpp<0xB1>(__float_as_uint(x)));
  x = mx(x, dpp<0x4E>(__float_as_uint(x)));
  x = mx(x, dpp<0x141>(__float_as_uint(x)));
  x = mx(x, dpp<0x140>(__float_as_uint(x)));
  x = mx(x, swz_xor16(__float_as_uint(x)));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <typename T, int D, int G>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int kvh, float (&qv)[G][8], float mul) {
  constexpr int LPR = D / 8;
  const int e = threadIdx.x % LPR;
  const T* q = (const T*)a.q + ((int64_t)b * a.Hq + kvh * G) * D + 8 * e;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Vec8<T> x;
    x.load(q + g * D);
    x.get(qv[g]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[g][i] *= mul;
  }
}

// key_out(r, orderable(max over the G heads of q . row r)) for rows [0, n) given by
// row_src(r), NP rows per thread in flight per round.
template <typename T, int D, int G, int NP, typename RowSrc, typename KeyOut>
__device__ __forceinline__ void score_rows(const float (&qv)[G][8], int n, const RowSrc& row_src,
                                           const KeyOut& key_out) {
  constexpr int LPR = D / 8, RPP = kDecThreads / LPR;
  const int tid = threadIdx.x, e = tid % LPR, rr = tid / LPR;
  for (int r0 = 0; r0 < n; r0 += NP * RPP) {
    Vec8<T> x[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = r0 + p * RPP + rr;
      if (r < n) x[p].load(row_src(r) + 8 * e);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = r0 + p * RPP + rr;
      float f[8];
      x[p].get(f);
      float best = -INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(qv[g][i], f[i], s);
        best = fmaxf(best, row_sum<LPR>(s));
      }
      if (e == 0 && r < n) key_out(r, score_key(best));
    }
  }
}

struct RouteShared {
  uint32_t ckeys[kSliceChunks];  // this work-group's chunk scores
  uint32_t gkeys[kMaxGroupCand + 4];
  int csel[64];
  int gsel[kMaxGroupCand];
  uint32_t cscr[64];             // score keys of csel
  TopkShared<kDecThreads> top;
  int nsel, flag;
};

// Top-k_g of the group keys[0 .. n) (n <= 512), ascending slots (= ascending group ids).
template <int P>
__device__ __forceinline__ int select_groups(RouteShared& sm, int n, int kg, int* out) {
  return wave_topk_sorted<P>(sm.gkeys, n, kg, out, &sm.nsel);
}

// ---------------------------------------------------------------- routing
template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_route_kernel(DecodeArgs a) {
  constexpr int NPR = sizeof(T) == 2 ? 4 : 2;   // rows per thread in flight (16 B each)
  __shared__ __align__(16) RouteShared sm;
  const int unit = blockIdx.x % a.n_units, slice = blockIdx.x / a.n_units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int p = a.pos[b];
  const bool active = p >= 0 && p < a.t_cap;
  const int J = active ? p / kChunk : 0;
  const int tid = threadIdx.x;
  const int64_t n_chunks = a.t_cap / kChunk;
  const T* cs = (const T*)a.csum + (int64_t)unit * n_chunks * D;
  const T* gs = (const T*)a.gsum + (int64_t)unit * (a.t_cap / kGroup) * D;
  uint64_t* cands = a.cands + (int64_t)unit * a.n_slices * a.kc;

  // ---- every work-group: its 64 candidate chunks, keeping their best k_c
  float qv[G][8];
  const int c0 = slice * kSliceChunks;
  if (c0 < J && a.kc > 0) {
    const int nrows = min(kSliceChunks, J - c0);
    load_q<T, D, G>(a, b, kvh, qv, 1.0f);
    score_rows<T, D, G, NPR>(qv, nrows, [&](int r) { return cs + (int64_t)(c0 + r) * D; },
                             [&](int r, uint32_t key) { sm.ckeys[r] = key; });
    __syncthreads();
    if (tid < 64) {
      uint64_t v[1] = {tid < nrows ? cand(sm.ckeys[tid], c0 + tid) : 0};
      const int m = wave_select<1>(v, a.kc, sm.top.fin);
      if (tid < a.kc) put(cands + slice * a.kc + tid, tid < m ? sm.top.fin[tid] : 0ull);
    }
  }
  if (!arrive_last(a.rcount + unit, a.n_slices, &sm.flag)) return;

  // ---- the last work-group of the unit: top-k_c, group scores, top-k_g
  const int N = a.kc > 0 ? (J + kSliceChunks - 1) / kSliceChunks * a.kc : 0;
  const int nc = N == 0 ? 0 : topk64(sm.top, N, a.kc, sm.csel, sm.cscr, [&](int i) { return get(cands + i); });
  const int ng_cand = 8 * nc;
  if (ng_cand > 0 && a.kg > 0) {
    load_q<T, D, G>(a, b, kvh, qv, 1.0f);
    score_rows<T, D, G, 2 * NPR>(qv, ng_cand, [&](int r) { return gs + (int64_t)(8 * sm.csel[r >> 3] + (r & 7)) * D; },
                           [&](int r, uint32_t key) { sm.gkeys[r] = key; });
  }
  __syncthreads();
  const int ng = (ng_cand == 0 || a.kg == 0) ? 0
                 : ng_cand <= 64            ? select_groups<1>(sm, ng_cand, a.kg, sm.gsel)
                 : ng_cand <= 128           ? select_groups<2>(sm, ng_cand, a.kg, sm.gsel)
                 : ng_cand <= 256           ? select_groups<4>(sm, ng_cand, a.kg, sm.gsel)
                                            : select_groups<8>(sm, ng_cand, a.kg, sm.gsel);
  if (a.cidx != nullptr) {
    for (int i = tid; i < a.kc; i += kDecThreads) {
      a.cidx[(int64_t)unit * a.kc + i] = i < nc ? sm.csel[i] : -1;
      if (a.cscore) a.cscore[(int64_t)unit * a.kc + i] = i < nc ? key_score(sm.cscr[i]) : -INFINITY;
    }
  }
  for (int i = tid; i < a.kg; i += kDecThreads) {
    const int slot = i < ng ? sm.gsel[i] : 0;
    a.gidx[(int64_t)unit * a.kg + i] = i < ng ? 8 * sm.csel[slot >> 3] + (slot & 7) : -1;
    if (a.gscore) a.gscore[(int64_t)unit * a.kg + i] = i < ng ? key_score(sm.gkeys[slot]) : -INFINITY;
  }
}

// ---------------------------------------------------------------- attention
template <typename T, int D, int G>
struct AttendShared {
  float s[G][kChunk];                 // logits, then probabilities
  float red[kDecWaves][G][D];         // cross-wave sum of P V
  float ml[G][2];                     // max and sum per head (log2 domain)
  int gid[kSplitGroups];              // this split's groups
  float wm[1 + kMaxGroupCand / kSplitGroups][G];   // merge: max, then weight, per split
  float wl[1 + kMaxGroupCand / kSplitGroups][G];   // merge: sum per split
  __align__(16) T ktile[kChunk][D];   // the own chunk's keys (summary update)
  float gs[8][D];                     // unscaled group sums of a completed chunk
  int flag;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_attend_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8, RPP = kDecThreads / LPR, NP = kChunk / RPP;   // passes over 64 tokens
  constexpr int PART = G * (D + 2);
  __shared__ __align__(16) AttendShared<T, D, G> sm;
  const int unit = blockIdx.x % a.n_units, split = blockIdx.x / a.n_units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int p = a.pos[b];
  const bool active = p >= 0 && p < a.t_cap;
  const int J = active ? p / kChunk : 0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e = tid % LPR, rr = tid / LPR;
  const T* kb = (const T*)a.k + (int64_t)unit * a.t_cap * D;
  const T* vb = (const T*)a.v + (int64_t)unit * a.t_cap * D;

  // Tokens of this split: split 0 = own chunk 64J .. p; split s = the valid ids among
  // selected groups 8(s-1) .. 8s-1 (an id outside [0, 8J) is skipped, so no read
  // leaves the history).
  if (w == 0) {
    int g = -1;
    const int slot = kSplitGroups * (split - 1) + lane;
    if (active && split > 0 && lane < kSplitGroups && slot < a.kg) g = a.gidx_in[(int64_t)unit * a.kg + slot];
    const bool ok = g >= 0 && g < kGroup * J;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
    if (ok) sm.gid[lanes_below(m)] = g;
    if (lane == 0) sm.flag = __builtin_popcountll(m);
  }
  __syncthreads();
  const int n_tok = !active ? 0 : split == 0 ? p - kChunk * J + 1 : kGroup * sm.flag;
  __syncthreads();
  auto tok_pos = [&](int i) __attribute__((always_inline)) -> int64_t {
    return split == 0 ? (int64_t)kChunk * J + i : (int64_t)kGroup * sm.gid[i / kGroup] + (i % kGroup);
  };

  float* part = a.part + ((int64_t)unit * a.n_split + split) * PART;
  if (n_tok > 0) {
    float qv[G][8];
    load_q<T, D, G>(a, b, kvh, qv, a.scale_log2);
    Vec8<T> kx[NP], vx[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int i = pp * RPP + rr;
      if (i < n_tok) {
        const int64_t t = tok_pos(i);
        kx[pp].load(kb + t * D + 8 * e);
        vx[pp].load(vb + t * D + 8 * e);
      }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int i = pp * RPP + rr;
      float f[8];
      kx[pp].get(f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(qv[g][c], f[c], s);
        s = row_sum<LPR>(s);
        if (e == 0) sm.s[g][i] = i < n_tok ? s : -INFINITY;
      }
    }
    __syncthreads();
    for (int g = w; g < G; g += kDecWaves) {   // softmax pieces of head g (one token per lane)
      const float x = sm.s[g][lane];
      const float m = wave_max(x);              // finite: split holds a valid token
      const float pe = x == -INFINITY ? 0.f : fast_exp2(x - m);
      const float l = wave_sum(pe);
      sm.s[g][lane] = pe;
      if (lane == 0) { sm.ml[g][0] = m; sm.ml[g][1] = l; }
    }
    __syncthreads();
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int i = pp * RPP + rr;
      float f[8];
      vx[pp].get(f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pv = sm.s[g][i];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(pv, f[c], acc[g][c]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] = col_sum<LPR>(acc[g][c]);
    if (lane < LPR) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) sm.red[w][g][8 * e + c] = acc[g][c];
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kDecThreads) {
      const int g = idx / D, dd = idx % D;
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < kDecWaves; ++ww) x += sm.red[ww][g][dd];
      put(part + idx, x);
    }
    if (tid < G) {
      put(part + G * D + tid, sm.ml[tid][0]);
      put(part + G * D + G + tid, sm.ml[tid][1]);
    }

    // Incremental summaries: the token completes its chunk.
    if (split == 0 && n_tok == kChunk && a.gsum_out != nullptr) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int i = pp * RPP + rr;
        float f[8];
        kx[pp].get(f);
#pragma unroll
        for (int c = 0; c < 8; ++c) store_elem(&sm.ktile[i][8 * e + c], f[c]);
      }
      __syncthreads();
      constexpr int TPG = D / 4;   // threads per group, 4 columns each
      const int gg = tid / TPG, cq = tid % TPG;
      if (gg < 8) {
        T* gout = (T*)a.gsum_out + ((int64_t)unit * (a.t_cap / kGroup) + 8 * J + gg) * D + 4 * cq;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float col[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) col[r] = widen(sm.ktile[8 * gg + r][4 * cq + c]);
          const float s = tree8(col);
          sm.gs[gg][4 * cq + c] = s;
          store_elem(gout + c, s * 0.125f);
        }
      }
      __syncthreads();
      if (tid < D) {
        float col[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) col[u] = sm.gs[u][tid];
        store_elem((T*)a.csum_out + ((int64_t)unit * (a.t_cap / kChunk) + J) * D + tid, tree8(col) * 0.015625f);
      }
    }
  } else if (tid < G) {
    put(part + G * D + tid, -INFINITY);   // empty split
    put(part + G * D + G + tid, 0.f);
  }
  if (!arrive_last(a.acount + unit, a.n_split, &sm.flag)) return;

  // ---- the last work-group of the unit merges the partials: per (split, head) the
  // weight 2^(m_s - M) / L, then O = sum of weight * O_s (8 splits' loads in flight)
  T* o = (T*)a.o + ((int64_t)b * a.Hq + kvh * G) * D;
  float* lse = a.lse + (int64_t)b * a.Hq + kvh * G;
  if (!active) {
    for (int idx = tid; idx < G * D; idx += kDecThreads) store_elem(o + idx, 0.f);
    if (tid < G) lse[tid] = -INFINITY;
    return;
  }
  const float* pu = a.part + (int64_t)unit * a.n_split * PART;
  constexpr int OPT = (G * D + kDecThreads - 1) / kDecThreads;   // outputs per thread
  constexpr int SB = 16;                                          // splits per round of loads
  float ov[SB][OPT];                                              // the first SB splits' O values
#pragma unroll
  for (int u = 0; u < SB; ++u)
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int idx = tid + j * kDecThreads;
      ov[u][j] = u < a.n_split && idx < G * D ? get(pu + u * PART + idx) : 0.f;
    }
  for (int i = tid; i < a.n_split * G; i += kDecThreads) {
    const int s2 = i / G, g = i % G;
    sm.wm[s2][g] = get(pu + s2 * PART + G * D + g);
    sm.wl[s2][g] = get(pu + s2 * PART + G * D + G + g);
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
    for (int s2 = 0; s2 < a.n_split; ++s2) M = fmaxf(M, sm.wm[s2][tid]);
    for (int s2 = 0; s2 < a.n_split; ++s2) {
      const float l = sm.wl[s2][tid];
      const float wgt = l > 0.f ? fast_exp2(sm.wm[s2][tid] - M) : 0.f;
      sm.wm[s2][tid] = wgt;
      L = fmaf(wgt, l, L);
    }
    for (int s2 = 0; s2 < a.n_split; ++s2) sm.wm[s2][tid] /= L;
    lse[tid] = (M + __log2f(L)) * kLn2;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int idx = tid + j * kDecThreads;
    if (idx >= G * D) break;
    const int g = idx / D;
    float x = 0.f;
#pragma unroll
    for (int u = 0; u < SB; ++u) x = u < a.n_split ? fmaf(sm.wm[u][g], ov[u][j], x) : x;
    for (int s0 = SB; s0 < a.n_split; s0 += SB) {
      float y[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) y[u] = s0 + u < a.n_split ? get(pu + (s0 + u) * PART + idx) : 0.f;
#pragma unroll
      for (int u = 0; u < SB; ++u) x = s0 + u < a.n_split ? fmaf(sm.wm[s0 + u][g], y[u], x) : x;
    }
    store_elem(o + idx, x);
  }
}

template <typename T, int D>
hipError_t launch_route_t(const DecodeArgs& a, int G, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_units * a.n_slices)), block(kDecThreads);
  switch (G) {
    case 1: return launch_kernel(decode_route_kernel<T, D, 1>, grid, block, s, a);
    case 2: return launch_kernel(decode_route_kernel<T, D, 2>, grid, block, s, a);
    case 4: return launch_kernel(decode_route_kernel<T, D, 4>, grid, block, s, a);
    default: return launch_kernel(decode_route_kernel<T, D, 8>, grid, block, s, a);
  }
}

template <typename T, int D>
hipError_t launch_attend_t(const DecodeArgs& a, int G, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_units * a.n_split)), block(kDecThreads);
  switch (G) {
    case 1: return launch_kernel(decode_attend_kernel<T, D, 1>, grid, block, s, a);
    case 2: return launch_kernel(decode_attend_kernel<T, D, 2>, grid, block, s, a);
    case 4: return launch_kernel(decode_attend_kernel<T, D, 4>, grid, block, s, a);
    default: return launch_kernel(decode_attend_kernel<T, D, 8>, grid, block, s, a);
  }
}

// Workspace: rcount, acount, keys, part (256-byte aligned pieces).
struct DecodeWs {
  size_t rcount, acount, keys, part, total;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// Workspace layout: the two arrival-counter arrays first (counter_slots entries
// each, at least one per unit), then the candidates and the partials.
DecodeWs decode_ws(const Dims& d, size_t counter_slots) {
  const size_t units = (size_t)d.B * d.Hkv;
  const size_t slots = counter_slots > units ? counter_slots : units;
  const size_t n_split = 1 + (d.kg + kSplitGroups - 1) / kSplitGroups;
  DecodeWs w;
  w.rcount = 0;
  w.acount = align256(slots * 4);
  w.keys = w.acount + align256(slots * 4);
  const size_t n_slices = (size_t)((d.t_cap / kChunk + kSliceChunks - 1) / kSliceChunks);
  w.part = w.keys + align256(units * n_slices * (size_t)d.kc * 8);
  w.total = w.part + align256(units * n_split * (size_t)d.G * (d.D + 2) * 4);
  return w;
}

DecodeArgs make_args(const Dims& d, void* ws, size_t counter_slots) {
  DecodeArgs a = {};
  const DecodeWs l = decode_ws(d, counter_slots);
  char* base = (char*)ws;
  a.rcount = (uint32_t*)(base + l.rcount);
  a.acount = (uint32_t*)(base + l.acount);
  a.cands = (uint64_t*)(base + l.keys);
  a.part = (float*)(base + l.part);
  a.t_cap = d.t_cap;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kc = d.kc; a.kg = d.kg;
  a.n_units = d.B * d.Hkv;
  a.n_slices = (int)((d.t_cap / kChunk + kSliceChunks - 1) / kSliceChunks);
  a.n_split = 1 + (d.kg + kSplitGroups - 1) / kSplitGroups;
  a.scale_log2 = d.scale * kLog2e;
  return a;
}

}  // namespace

size_t decode_workspace_bytes(const Dims& d, size_t counter_slots) { return decode_ws(d, counter_slots).total; }
size_t decode_counter_bytes(size_t counter_slots) { return 2 * align256(counter_slots * 4); }

hipError_t launch_decode(const Dims& d, bool bf16, bool route, bool attend, const void* q, const void* k,
                         const void* v, const void* chunk_sum, const void* group_sum, const int32_t* pos,
                         int32_t* chunk_idx, int32_t* group_idx, float* chunk_score, float* group_score,
                         void* o, float* lse, void* group_sum_out, void* chunk_sum_out, void* ws,
                         hipStream_t s, size_t counter_slots) {
  DecodeArgs a = make_args(d, ws, counter_slots);
  a.q = q; a.k = k; a.v = v; a.csum = chunk_sum; a.gsum = group_sum; a.pos = pos;
  a.cidx = chunk_idx; a.gidx = group_idx; a.gidx_in = group_idx; a.cscore = chunk_score; a.gscore = group_score;
  a.o = o; a.lse = lse; a.gsum_out = group_sum_out; a.csum_out = chunk_sum_out;
  hipError_t e = hipSuccess;
  if (route) {
    e = bf16 ? (d.D == 128 ? launch_route_t<uint16_t, 128>(a, d.G, s) : launch_route_t<uint16_t, 64>(a, d.G, s))
             : (d.D == 128 ? launch_route_t<float, 128>(a, d.G, s) : launch_route_t<float, 64>(a, d.G, s));
    if (e != hipSuccess) return e;
  }
  if (attend) {
    e = bf16 ? (d.D == 128 ? launch_attend_t<uint16_t, 128>(a, d.G, s) : launch_attend_t<uint16_t, 64>(a, d.G, s))
             : (d.D == 128 ? launch_attend_t<float, 128>(a, d.G, s) : launch_attend_t<float, 64>(a, d.G, s));
  }
  return e;
}

}  // namespace hga
