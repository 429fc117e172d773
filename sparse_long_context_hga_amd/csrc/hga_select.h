// Exact top-k selection of a work-group over orderable score keys (ties go to
// the lower index; the result is written in ascending index order).  Used by the
// routing kernels of the segment path and of the generation path.
#pragma once

#include "hga_device.h"

namespace hga {
namespace {

constexpr int kRouteThreads = 512;      // threads of the segment path's bf16 routing work-groups
constexpr int kRouteThreadsF32 = 256;   // and of its fp32 ones
constexpr int kMaxChunks = 8192;     // = HGA_MAX_CHUNKS
constexpr int kMaxGroupCand = 512;   // 8 * max top_chunks

// NT: threads of the calling work-group (a multiple of 64, at least 256).
template <int NT>
struct SelectShared {
  uint32_t hist[256];
  int scan[NT / 64];
  int digit, above;
};

// Indices of the k largest keys[0..n) (ties -> lower index), written ascending to
// out[0..min(k,n)).  Keys must be distinct from 0 for real candidates.  Returns
// the number written.  All threads of the block must call it.
template <int NT>
__device__ int block_topk(const uint32_t* keys, int n, int k, int* out, SelectShared<NT>& sh) {
  static_assert(NT >= 256 && NT % 64 == 0, "one thread per digit");
  const int tid = threadIdx.x;
  if (k <= 0 || n <= 0) return 0;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) out[i] = i;
    __syncthreads();
    return n;
  }
  uint32_t prefix = 0, pmask = 0;
  int kk = k;  // rank (1-based) of the k-th key among keys matching `prefix`
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Suffix sums over digits: thread t looks at digit 255 - t.
    const int hv = tid < 256 ? (int)sh.hist[255 - tid] : 0;
    int tot;
    const int ex = block_exclusive_scan<NT>(hv, sh.scan, tot);  // keys in higher digits
    if (tid < 256 && ex < kk && kk <= ex + hv) {
      sh.digit = 255 - tid;
      sh.above = ex;
    }
    __syncthreads();
    prefix |= ((uint32_t)sh.digit) << shift;
    pmask |= 255u << shift;
    kk -= sh.above;
    __syncthreads();
  }
  // Threshold key T = prefix: take every key > T and the kk lowest-index keys == T.
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per, hi = min(n, lo + per);
  int n_eq = 0;
  for (int i = lo; i < hi; ++i) n_eq += keys[i] == prefix;
  int tot;
  int eq_before = block_exclusive_scan<NT>(n_eq, sh.scan, tot);
  int n_sel = 0;
  {
    int e = eq_before;
    for (int i = lo; i < hi; ++i) {
      const uint32_t u = keys[i];
      if (u > prefix) ++n_sel;
      else if (u == prefix) { n_sel += e < kk; ++e; }
    }
  }
  int sel_before = block_exclusive_scan<NT>(n_sel, sh.scan, tot);
  {
    int e = eq_before, o = sel_before;
    for (int i = lo; i < hi; ++i) {
      const uint32_t u = keys[i];
      bool take = false;
      if (u > prefix) take = true;
      else if (u == prefix) { take = e < kk; ++e; }
      if (take) out[o++] = i;
    }
  }
  __syncthreads();
  return k;
}

// ---------------------------------------------------------------- one-wave selection
// Candidates for the selection: score key << 32 | (2^32 - 1 - index), so that a
// larger value is a higher score or, at equal score, a lower index; 0 = none.
__device__ __forceinline__ uint64_t cand(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int cand_index(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }
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
    if (cnt >= k) {
      res = t;
      if (cnt == k) break;   // exactly k at or above: any larger threshold keeps the same set
    }
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

// Wave 0 of the calling work-group selects the top k (k >= 1) of keys[0 .. n)
// (n <= 64 P; keys nonzero) by (key desc, index asc) and stores their indices in
// ascending order to out.  Lane l holds the candidates P l .. P l + P - 1, so the
// selected ones of the lanes below come first: their count is a prefix sum, taken
// from bit-sliced ballots.  Returns the number selected (all threads; sm_n: LDS).
template <int P>
__device__ __forceinline__ int wave_topk_sorted(const uint32_t* keys, int n, int k, int* out, int* sm_n) {
  static_assert(P <= 8, "counts of at most 15 per lane");
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint64_t v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int s = P * lane + i;
      v[i] = s < n ? cand(keys[s], s) : 0;
    }
    const uint64_t th = wave_kth<P>(v, k);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) cnt += v[i] != 0 && v[i] >= th;
    int before = 0;
#pragma unroll
    for (int bit = 0; bit < 4; ++bit) before += lanes_below(__builtin_amdgcn_ballot_w64((cnt >> bit) & 1)) << bit;
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (v[i] != 0 && v[i] >= th) out[before++] = P * lane + i;
    if (lane == 63) *sm_n = before;
  }
  __syncthreads();
  return *sm_n;
}

// ---------------------------------------------------------------- top-k of at most 64, any n
// Scratch of topk64 for a work-group of NT threads.
template <int NT>
struct TopkShared {
  uint64_t win[NT];   // each wave's best k (k <= 64)
  uint64_t fin[64];   // the selected candidates, any order
  int nsel;
};

// Lanes n' < n of the calling wave: the candidates fin[0 .. n) (distinct chunk
// indices below kMaxChunks, any order) to out / out_keys (nullable) in ascending
// index order.  A candidate's slot is the number of candidates with a lower index,
// counted over the index bits with ballots, most significant first: at each bit, a
// lane whose bit is set adds the lanes that agree with it on the higher bits and
// have the bit clear.
constexpr int kIndexBits = 13;
static_assert(kMaxChunks <= (1 << kIndexBits), "chunk indices fit the counted bits");
__device__ __forceinline__ void sort_by_index(const uint64_t* fin, int n, int* out, uint32_t* out_keys) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < n;
  const uint64_t x = valid ? fin[lane] : 0ull;
  const uint32_t idx = valid ? (uint32_t)cand_index(x) : 0u;
  uint64_t same = __builtin_amdgcn_ballot_w64(valid);   // lanes agreeing with this one on the bits above b
  int rank = 0;
#pragma unroll
  for (int b = kIndexBits - 1; b >= 0; --b) {
    const bool one = (idx >> b) & 1u;
    const uint64_t ones = __builtin_amdgcn_ballot_w64(valid && one);
    if (one) rank += __builtin_popcountll(same & ~ones);
    same &= one ? ones : ~ones;
  }
  if (valid) {
    out[rank] = (int)idx;
    if (out_keys) out_keys[rank] = (uint32_t)(x >> 32);
  }
}

template <int NT, int P, typename F>
__device__ __forceinline__ int topk64_one_wave(TopkShared<NT>& sh, int n, int k, int* out, uint32_t* out_keys,
                                               const F& cand_at) {
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    uint64_t v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = lane + 64 * i < n ? cand_at(lane + 64 * i) : 0;
    const int m = wave_select<P>(v, k, sh.fin);
    sort_by_index(sh.fin, m, out, out_keys);
    if (lane == 0) sh.nsel = m;
  }
  __syncthreads();
  return sh.nsel;
}

// Every wave keeps the best k of its candidates (i = tid + NT p), then wave 0 selects
// among the waves' NW k (P2 per lane).
template <int NT, int P, int P2, typename F>
__device__ __forceinline__ int topk64_two_stage(TopkShared<NT>& sh, int n, int k, int* out, uint32_t* out_keys,
                                                const F& cand_at) {
  constexpr int NW = NT / 64;
  static_assert(64 * P2 >= NT, "room for every wave's best 64");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint64_t v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) v[i] = tid + NT * i < n ? cand_at(tid + NT * i) : 0;
  uint64_t* mine = sh.win + w * k;
  const int m = wave_select<P>(v, k, mine);
  for (int i = m + lane; i < k; i += 64) mine[i] = 0;
  __syncthreads();
  if (w == 0) {
    uint64_t u[P2];
#pragma unroll
    for (int q = 0; q < P2; ++q) u[q] = lane + 64 * q < NW * k ? sh.win[lane + 64 * q] : 0;
    const int m2 = wave_select<P2>(u, k, sh.fin);
    sort_by_index(sh.fin, m2, out, out_keys);
    if (lane == 0) sh.nsel = m2;
  }
  __syncthreads();
  return sh.nsel;
}

// Top-k (1 <= k <= 64) of the n candidates cand_at(i), i < n <= 32 NT (nonzero,
// distinct 64-bit candidate values, see cand), written to out (and their score keys
// to out_keys, nullable) in ascending index order.  Returns min(k, n); all threads
// of the work-group must call it.
template <int NT, typename F>
__device__ __forceinline__ int topk64(TopkShared<NT>& sh, int n, int k, int* out, uint32_t* out_keys,
                                      const F& cand_at) {
  static_assert(NT == 256 || NT == 512, "4 or 8 waves");
  constexpr int P2 = NT / 64;   // the waves' best k (<= 64 each), per lane of the final wave
  if (n <= 64) return topk64_one_wave<NT, 1>(sh, n, k, out, out_keys, cand_at);
  if (n <= 128) return topk64_one_wave<NT, 2>(sh, n, k, out, out_keys, cand_at);
  if (n <= 256) return topk64_one_wave<NT, 4>(sh, n, k, out, out_keys, cand_at);
  if (n <= 512) return topk64_one_wave<NT, 8>(sh, n, k, out, out_keys, cand_at);
  if (n <= NT * 2) return topk64_two_stage<NT, 2, P2>(sh, n, k, out, out_keys, cand_at);
  if (n <= NT * 4) return topk64_two_stage<NT, 4, P2>(sh, n, k, out, out_keys, cand_at);
  if (n <= NT * 8) return topk64_two_stage<NT, 8, P2>(sh, n, k, out, out_keys, cand_at);
  if (n <= NT * 16) return topk64_two_stage<NT, 16, P2>(sh, n, k, out, out_keys, cand_at);
  return topk64_two_stage<NT, 32, P2>(sh, n, k, out, out_keys, cand_at);
}

}  // namespace
}  // namespace hga
