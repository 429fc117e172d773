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
// One work-group of 512 threads per (sequence, KV head): a decode step has little
// work per unit and nothing to share between units, so the unit's whole chain --
// chunk scores, top-k_c, group scores, top-k_g, attention, summary update -- runs
// in one work-group with its intermediate results in LDS, and a step is one
// launch.  Rows (summaries, keys, values) are read by D/8 lanes each, 16 B per
// lane, many rows in flight per thread; scores and attention are G-row GEMVs on
// the vector ALUs in fp32 (not GEMM-shaped, so no MFMA).  Attention walks the key
// list in tiles with an online softmax per head.
#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"

#include <math.h>

namespace hga {
namespace {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;

enum : int { kRoute = 1, kAttend = 2 };

struct DecodeArgs {
  const void* q;          // [B, Hq, d]
  const void* k;          // [B, Hkv, t_cap, d]
  const void* v;
  const void* csum;       // [B, Hkv, t_cap/64, d]
  const void* gsum;       // [B, Hkv, t_cap/8, d]
  void* csum_out;         // summary tables updated by the attention (nullable)
  void* gsum_out;
  const int32_t* pos;     // [B]
  int32_t* cidx;          // [B, Hkv, k_c] (nullable in a fused step)
  int32_t* gidx;          // [B, Hkv, k_g]
  const int32_t* gidx_in; // attention only: the selection to attend
  float* cscore;
  float* gscore;
  void* o;                // [B, Hq, d]
  float* lse;             // [B, Hq]
  int64_t t_cap;
  int Hq, Hkv, kc, kg, n_units;
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

// Candidates for the selection: score key << 32 | (2^32 - 1 - index), so that a
// larger value is a higher score or, at equal score, a lower index; 0 = none.
__device__ __forceinline__ uint64_t cand(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int cand_index(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  return ((uint64_t)dpp<CTRL>((uint32_t)(x >> 32)) << 32) | dpp<CTRL>((uint32_t)x);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = umax64(x, dpp64<0xB1>(x));
  x = umax64(x, dpp64<0x4E>(x));
  x = umax64(x, dpp64<0x141>(x));
  x = umax64(x, dpp64<0x140>(x));
  x = umax64(x, ((uint64_t)swz_xor16((uint32_t)(x >> 32)) << 32) | swz_xor16((uint32_t)x));
  const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return umax64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
}

// The k-th largest of the wave's candidates v[P] (P per lane), or 0 when the wave
// holds at most k: a most-significant-bit-first search on the 64-bit values,
// counting with ballots (the counts are wave-uniform scalars).  Candidates are
// distinct, so exactly min(k, #candidates) of them are >= the result and nonzero.
template <int P>
__device__ __forceinline__ uint64_t wave_kth(const uint64_t (&v)[P], int k) {
  uint64_t res = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t t = res | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[i] >= t));
    if (cnt >= k) res = t;
  }
  return res;
}

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Selects the k largest of the wave's candidates (k >= 1) and stores them to out
// in an order fixed by (lane, i); returns their number (wave-uniform).
template <int P>
__device__ __forceinline__ int wave_select(const uint64_t (&v)[P], int k, uint64_t* out) {
  const uint64_t th = wave_kth<P>(v, k);
  int base = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const bool sel = v[i] != 0 && v[i] >= th;
    const uint64_t m = __builtin_amdgcn_ballot_w64(sel);
    if (sel) out[base + lanes_below(m)] = v[i];
    base += __builtin_popcountll(m);
  }
  return base;
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

// key[r] = orderable(max over the G heads of q . row r) for rows [0, n) given by
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

template <typename T, int D, int G>
struct DecodeShared {
  static constexpr int LPR = D / 8, RPP = kDecThreads / LPR;
  static constexpr int NPA = sizeof(T) == 2 ? 8 : 4;        // attention rows per thread per tile
  static constexpr int TT = NPA * RPP;                       // tokens per attention tile
  uint32_t ckeys[kMaxChunks + 4];
  uint32_t gkeys[kMaxGroupCand + 4];
  int csel[64];
  int gsel[kMaxGroupCand];      // route: selected slots; attention: the group ids to attend
  float s[G][TT];               // logits, then probabilities, of one tile
  float alpha[G];               // rescale of the running output per head
  float red[kDecWaves][G][D];   // cross-wave sum of P V
  float stat[G][2];             // running max and sum per head (log2 domain)
  float gs[8][D];               // unscaled group sums of a completed chunk
  uint64_t win[kDecWaves * 64]; // each wave's best chunk candidates (k_c per wave)
  uint64_t fin[64];             // the selected chunks, best first
  int nsel;
};

// Top-k_c (1 <= k_c <= 64) of the chunk keys[0 .. J): each wave selects the best
// k_c of the chunks c = tid + 512 i its lanes own (P per lane), wave 0 the best k_c
// of those (P2 per lane), stored in ascending chunk order to csel.  Returns their
// number (all threads).
template <int P, int P2, typename S>
__device__ __forceinline__ int select_chunks(S& sm, int J, int kc) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint64_t v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int c = tid + kDecThreads * i;
    v[i] = c < J ? cand(sm.ckeys[c], c) : 0;
  }
  uint64_t* mine = sm.win + w * kc;
  const int m = wave_select<P>(v, kc, mine);
  for (int i = m + lane; i < kc; i += 64) mine[i] = 0;
  __syncthreads();
  if (w == 0) {
    uint64_t u[P2];
#pragma unroll
    for (int q = 0; q < P2; ++q) {
      const int i = lane + 64 * q;
      u[q] = i < kDecWaves * kc ? sm.win[i] : 0;
    }
    const int n = wave_select<P2>(u, kc, sm.fin);
    if (lane < n) {
      const int idx = cand_index(sm.fin[lane]);
      int rank = 0;
      for (int j = 0; j < n; ++j) rank += cand_index(sm.fin[j]) < idx;
      sm.csel[rank] = idx;
    }
    if (lane == 0) sm.nsel = n;
  }
  __syncthreads();
  return sm.nsel;
}

template <int P, typename S>
__device__ __forceinline__ int select_chunks_p(S& sm, int J, int kc) {
  if (kc <= 8) return select_chunks<P, 1>(sm, J, kc);
  if (kc <= 16) return select_chunks<P, 2>(sm, J, kc);
  if (kc <= 32) return select_chunks<P, 4>(sm, J, kc);
  return select_chunks<P, 8>(sm, J, kc);
}

// Top-k_g of the group keys[0 .. n) (n <= 512) by wave 0, stored in ascending slot
// order (= ascending group id) to out.  Returns their number (all threads).
template <int P, typename S>
__device__ __forceinline__ int select_groups(S& sm, int n, int kg, int* out) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (w == 0) {
    uint64_t v[P];   // lane l holds slots P l .. P l + P - 1
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int s = P * lane + i;
      v[i] = s < n ? cand(sm.gkeys[s], s) : 0;
    }
    const uint64_t th = wave_kth<P>(v, kg);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) cnt += v[i] != 0 && v[i] >= th;
    int before = 0;   // selected slots of the lanes below: bit-sliced ballots of cnt (< 16)
#pragma unroll
    for (int bit = 0; bit < 4; ++bit) before += lanes_below(__builtin_amdgcn_ballot_w64((cnt >> bit) & 1)) << bit;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (v[i] != 0 && v[i] >= th) out[before++] = P * lane + i;
    }
    if (lane == 63) sm.nsel = before;
  }
  __syncthreads();
  return sm.nsel;
}

template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  using S = DecodeShared<T, D, G>;
  constexpr int LPR = S::LPR, RPP = S::RPP, NPA = S::NPA, TT = S::TT;
  constexpr int NPR = sizeof(T) == 2 ? 16 : 8;               // scoring rows per thread in flight
  __shared__ __align__(16) S sm;

  const int unit = blockIdx.x;
  if (unit >= a.n_units) return;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int p = a.pos[b];
  const bool active = p >= 0 && p < a.t_cap;
  const int J = active ? p / kChunk : 0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e = tid % LPR, rr = tid / LPR;

  // ---------------------------------------------------------------- routing
  int ng = 0;   // groups to attend (their ids in sm.gsel[0 .. ng))
  if constexpr ((MODE & kRoute) != 0) {
    const int64_t n_chunks = a.t_cap / kChunk;
    const T* cs = (const T*)a.csum + (int64_t)unit * n_chunks * D;
    const T* gs = (const T*)a.gsum + (int64_t)unit * (a.t_cap / kGroup) * D;
    float qv[G][8];
    if (J > 0) {
      load_q<T, D, G>(a, b, kvh, qv, 1.0f);
      score_rows<T, D, G, NPR>(qv, J, [&](int r) { return cs + (int64_t)r * D; },
                               [&](int r, uint32_t key) { sm.ckeys[r] = key; });
    }
    __syncthreads();
    const int nc = (J == 0 || a.kc == 0) ? 0
                   : J <= kDecThreads     ? select_chunks_p<1>(sm, J, a.kc)
                   : J <= 4 * kDecThreads ? select_chunks_p<4>(sm, J, a.kc)
                                          : select_chunks_p<16>(sm, J, a.kc);
    const int ng_cand = 8 * nc;
    if (ng_cand > 0)
      score_rows<T, D, G, 4>(qv, ng_cand,
                             [&](int r) { return gs + (int64_t)(8 * sm.csel[r >> 3] + (r & 7)) * D; },
                             [&](int r, uint32_t key) { sm.gkeys[r] = key; });
    __syncthreads();
    ng = (ng_cand == 0 || a.kg == 0) ? 0
         : ng_cand <= 64  ? select_groups<1>(sm, ng_cand, a.kg, sm.gsel)
         : ng_cand <= 128 ? select_groups<2>(sm, ng_cand, a.kg, sm.gsel)
         : ng_cand <= 256 ? select_groups<4>(sm, ng_cand, a.kg, sm.gsel)
                          : select_groups<8>(sm, ng_cand, a.kg, sm.gsel);   // ascending slots = ascending ids
    if (a.cidx != nullptr) {
      for (int i = tid; i < a.kc; i += kDecThreads) {
        a.cidx[(int64_t)unit * a.kc + i] = i < nc ? sm.csel[i] : -1;
        if (a.cscore) a.cscore[(int64_t)unit * a.kc + i] = i < nc ? key_score(sm.ckeys[sm.csel[i]]) : -INFINITY;
      }
    }
    // slots -> group ids, in place (each thread rewrites the entries it reads)
    int gid[kMaxGroupCand / kDecThreads + 1];
    float gsc[kMaxGroupCand / kDecThreads + 1];
#pragma unroll
    for (int u = 0; u * kDecThreads < kMaxGroupCand; ++u) {
      const int i = tid + u * kDecThreads;
      const int slot = i < ng ? sm.gsel[i] : 0;
      gid[u] = 8 * sm.csel[slot >> 3] + (slot & 7);
      gsc[u] = key_score(sm.gkeys[slot]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u * kDecThreads < kMaxGroupCand; ++u) {
      const int i = tid + u * kDecThreads;
      if (i < ng) sm.gsel[i] = gid[u];
      if (i < a.kg && a.gidx != nullptr) {
        a.gidx[(int64_t)unit * a.kg + i] = i < ng ? gid[u] : -1;
        if (a.gscore) a.gscore[(int64_t)unit * a.kg + i] = i < ng ? gsc[u] : -INFINITY;
      }
    }
    __syncthreads();
  } else {
    // the selection to attend, as the routing writes it: valid ids (before the own
    // chunk) first, then -1; anything else ends the list, so no read leaves the history
    if (active) {
      for (int i = tid; i < a.kg; i += kDecThreads) sm.gsel[i] = a.gidx_in[(int64_t)unit * a.kg + i];
    }
    __syncthreads();
    if (active) {
      while (ng < a.kg && sm.gsel[ng] >= 0 && sm.gsel[ng] < kGroup * J) ++ng;
    }
  }
  if constexpr ((MODE & kAttend) == 0) return;

  // ---------------------------------------------------------------- attention
  T* o = (T*)a.o + ((int64_t)b * a.Hq + kvh * G) * D;
  float* lse = a.lse + (int64_t)b * a.Hq + kvh * G;
  if (!active) {
    for (int i = tid; i < G * D; i += kDecThreads) store_elem(o + i, 0.f);
    if (tid < G) lse[tid] = -INFINITY;
    return;
  }
  const T* kb = (const T*)a.k + (int64_t)unit * a.t_cap * D;
  const T* vb = (const T*)a.v + (int64_t)unit * a.t_cap * D;
  const int n_sel = kGroup * ng;
  const int n_tok = n_sel + (p - kChunk * J + 1);
  auto tok_pos = [&](int i) __attribute__((always_inline)) -> int64_t {
    return i < n_sel ? (int64_t)kGroup * sm.gsel[i / kGroup] + (i % kGroup) : (int64_t)kChunk * J + (i - n_sel);
  };
  float qv[G][8];
  load_q<T, D, G>(a, b, kvh, qv, a.scale_log2);
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;    // wave g < G keeps head g's running statistics

  for (int t0 = 0; t0 < n_tok; t0 += TT) {
    Vec8<T> kx[NPA], vx[NPA];
#pragma unroll
    for (int pp = 0; pp < NPA; ++pp) {
      const int i = t0 + pp * RPP + rr;
      if (i < n_tok) {
        const int64_t t = tok_pos(i);
        kx[pp].load(kb + t * D + 8 * e);
        vx[pp].load(vb + t * D + 8 * e);
      }
    }
#pragma unroll
    for (int pp = 0; pp < NPA; ++pp) {
      const int i = t0 + pp * RPP + rr;
      float f[8];
      kx[pp].get(f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) s = fmaf(qv[g][c], f[c], s);
        s = row_sum<LPR>(s);
        if (e == 0) sm.s[g][pp * RPP + rr] = i < n_tok ? s : -INFINITY;
      }
    }
    __syncthreads();
    if (w < G) {   // online softmax of head w over this tile
      float x[TT / 64];
      float mt = -INFINITY;   // tile maximum
#pragma unroll
      for (int u = 0; u < TT / 64; ++u) {
        x[u] = sm.s[w][u * 64 + lane];
        mt = fmaxf(mt, x[u]);
      }
      mt = wave_max(mt);
      const float m_new = fmaxf(m_run, mt);          // finite: the tile holds a valid key
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < TT / 64; ++u) {
        const float pe = x[u] == -INFINITY ? 0.f : fast_exp2(x[u] - m_new);
        sm.s[w][u * 64 + lane] = pe;
        sum += pe;
      }
      sum = wave_sum(sum);
      const float al = fast_exp2(m_run - m_new);     // 0 on the first tile
      l_run = l_run * al + sum;
      m_run = m_new;
      if (lane == 0) sm.alpha[w] = al;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float al = sm.alpha[g];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] *= al;
    }
#pragma unroll
    for (int pp = 0; pp < NPA; ++pp) {
      float f[8];
      vx[pp].get(f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pv = sm.s[g][pp * RPP + rr];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(pv, f[c], acc[g][c]);
      }
    }
    __syncthreads();   // the next tile overwrites sm.s
  }
  if (w < G && lane == 0) {
    sm.stat[w][0] = m_run;
    sm.stat[w][1] = l_run;
  }
  // rows -> one value per (head, column): lanes of a wave first, then the waves
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
    store_elem(o + idx, x / sm.stat[g][1]);
  }
  if (tid < G) lse[tid] = (sm.stat[tid][0] + __log2f(sm.stat[tid][1])) * kLn2;

  // ---------------------------------------------------------------- summaries
  // The token completes its chunk: build the chunk's group and chunk summaries.
  if (a.gsum_out != nullptr && p % kChunk == kChunk - 1) {
    constexpr int TPG = D / 4;   // threads per group, 4 columns each
    const int gg = tid / TPG, cq = tid % TPG;
    if (gg < 8) {
      const T* kp = kb + ((int64_t)kChunk * J + kGroup * gg) * D + 4 * cq;
      T* gout = (T*)a.gsum_out + ((int64_t)unit * (a.t_cap / kGroup) + 8 * J + gg) * D + 4 * cq;
      float x[8][4];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) x[r][c] = widen(kp[(int64_t)r * D + c]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float col[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) col[r] = x[r][c];
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
}

template <typename T, int D, int MODE>
hipError_t launch_t(const DecodeArgs& a, int G, hipStream_t s) {
  const dim3 grid((unsigned)a.n_units), block(kDecThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<T, D, 1, MODE>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, D, 2, MODE>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, D, 4, MODE>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decode_kernel<T, D, 8, MODE>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const Dims& d, bool bf16, const DecodeArgs& a, hipStream_t s) {
  if (bf16) return d.D == 128 ? launch_t<uint16_t, 128, MODE>(a, d.G, s) : launch_t<uint16_t, 64, MODE>(a, d.G, s);
  return d.D == 128 ? launch_t<float, 128, MODE>(a, d.G, s) : launch_t<float, 64, MODE>(a, d.G, s);
}

DecodeArgs make_args(const Dims& d) {
  DecodeArgs a = {};
  a.t_cap = d.t_cap;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kc = d.kc; a.kg = d.kg;
  a.n_units = d.B * d.Hkv;
  a.scale_log2 = d.scale * kLog2e;
  return a;
}

}  // namespace

hipError_t launch_decode(const Dims& d, bool bf16, bool route, bool attend, const void* q, const void* k,
                         const void* v, const void* chunk_sum, const void* group_sum, const int32_t* pos,
                         int32_t* chunk_idx, int32_t* group_idx, float* chunk_score, float* group_score,
                         void* o, float* lse, void* group_sum_out, void* chunk_sum_out, hipStream_t s) {
  DecodeArgs a = make_args(d);
  a.q = q; a.k = k; a.v = v; a.csum = chunk_sum; a.gsum = group_sum; a.pos = pos;
  a.cidx = chunk_idx; a.gidx = group_idx; a.gidx_in = group_idx; a.cscore = chunk_score; a.gscore = group_score;
  a.o = o; a.lse = lse; a.gsum_out = group_sum_out; a.csum_out = chunk_sum_out;
  if (route && attend) return launch_mode<kRoute | kAttend>(d, bf16, a, s);
  if (route) return launch_mode<kRoute>(d, bf16, a, s);
  return launch_mode<kAttend>(d, bf16, a, s);
}

}  // namespace hga
