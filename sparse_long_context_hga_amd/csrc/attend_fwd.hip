// Exact attention over the selected groups' exact-token K/V plus the own chunk.
//
// Pages: seventnews "BMW如何通过重新设计注意力机制，在16 GB GPU上实现16K上下文", section
// "HGA的不同之处" (only the selected groups' exact K/V are loaded; summaries never
// act as values or outputs) and the adnankhan.ai note, section "Raw Abstract /
// Excerpt" (a bounded set of exact historical tokens per query block).  Reading
// of this library: each query also attends its own 64-token chunk causally.
//
// bf16 path, one work-group per (sequence, KV head, query block), 2G waves of
// 32 query rows each (the G query heads of the KV head share every gathered
// tile: GQA-aware, one gather per KV head):
//   * key tiles of 64 tokens: the own chunk first (its own buffer set), then 8
//     selected groups per tile (each group is one contiguous 2 KiB run of K and of
//     V in HBM) through two buffer sets in swizzled LDS, the next tile's copies in
//     flight during the MFMAs;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys in rho order, B = the
//     wave's 32 query rows held in registers): each lane ends with one query row
//     and 32 of the 64 keys, so the online-softmax statistics live in the lane;
//   * O^T += V^T P^T: P (bf16) is already in operand-B layout thanks to rho, and
//     V^T comes from the row-major tile through ds_read_b64_tr_b16.
// The same attention also runs right after the routing of the unit in one
// work-group (route_attend_bf16_kernel, 4 query heads per KV head): the query rows
// are loaded once for both, and the selection goes from LDS to the tile copies
// without a round trip through memory or a kernel boundary.
// fp32 path: one thread per query row, plain fp32 loops (exact-precision mode).
#include "hga_device.h"
#include "hga_internal.h"
#include "route_phase.h"

#include <math.h>

namespace hga {
namespace {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* gidx;
  void* o;
  float* lse;
  int64_t t_cap, t_hist, seg_len;
  int Hq, Hkv, kg, nb, n_units;
  float scale;
};

// Copies of the own chunk's 64 K and V rows of unit `unit` into tile buffers kt / vt
// (NW waves; asynchronous: the attention below waits for them).  The own chunk does
// not depend on the selection, so a caller issues them as early as it likes.
template <int D, int NW>
__device__ __forceinline__ void issue_own_tile(const FwdArgs& a, int unit, uint16_t* kt, uint16_t* vt) {
  const int j = unit % a.nb;
  const int bh = unit / a.nb;
  const int64_t row0 = (int64_t)bh * a.t_cap + (a.t_hist / kChunk + j) * kChunk;
  const uint16_t* kp = (const uint16_t*)a.k + row0 * D;
  const uint16_t* vp = (const uint16_t*)a.v + row0 * D;
  dma_tile<D, NW>(kt, [&](int r) { return kp + (int64_t)r * D; });
  dma_tile<D, NW>(vt, [&](int r) { return vp + (int64_t)r * D; });
}

// Attention of this work-group's HPW query heads of unit `unit` (head offset
// sub * HPW within the KV group) over its own chunk (causally) and the selected
// groups sgid[0 .. n_valid) (ascending, in LDS); qf: the lane's query row fragments
// (row n of the wave's 32).  KB(B) / VB(B) give the K / V tile buffer set B
// (distinct LDS arrays): the own chunk is tile 0, already in flight into set 2
// (issue_own_tile, the only copies this wave has outstanding); the selected groups
// follow, 8 per tile, through sets 0 and 1, which also serve as the waves' output
// regions at the end.
template <int D, int G, int HPW, typename KBuf, typename VBuf>
__device__ __forceinline__ void attend_unit_bf16(const FwdArgs& a, int unit, int sub, const bf16x8 (&qf)[D / 16],
                                                 const int* sgid, int n_valid, const KBuf& KB, const VBuf& VB) {
  constexpr int NW = 2 * HPW;
  constexpr int KS = D / 16;       // k-steps over the head dimension
  constexpr int DT = D / 32;       // 32-wide column tiles of O^T
  (void)KS;
  const int j = unit % a.nb;
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = l & 31;
  const int hh = sub * HPW + (w >> 1);    // query head within the KV group
  const int pos = 32 * (w & 1) + n;       // this lane's query position in the block
  // First row of this wave's 32 (wave-uniform) and this lane's row.
  const int64_t qrow0 = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)j * kQBlock + 32 * (w & 1);
  const int64_t qrow = qrow0 + n;

  const char* kb = (const char*)a.k + (int64_t)bh * a.t_cap * D * 2;
  const char* vb = (const char*)a.v + (int64_t)bh * a.t_cap * D * 2;
  // 32-row LDS region of wave wv in the first two tile buffer sets (for O after the
  // last tile).
  auto row_region = [&](int wv) __attribute__((always_inline)) -> uint16_t* {
    uint16_t* base = (wv >> 1) == 0 ? KB(ic<0>{}) : (wv >> 1) == 1 ? VB(ic<0>{}) : (wv >> 1) == 2 ? KB(ic<1>{})
                                                                                                : VB(ic<1>{});
    return base + (wv & 1) * 32 * D;
  };
  const int n_sel_tiles = (n_valid + 7) >> 3;
  const int n_tiles = n_sel_tiles + 1;

  // Groups of slot s (0..7) of selected tile t >= 1 (wave-uniform): groups
  // 8(t-1) .. of the selection; slots past it repeat the own chunk's first group
  // (masked later).
  GroupCopier<D, NW> copier;
  auto prepare = [&](int t_) __attribute__((always_inline)) {
    const int t = __builtin_amdgcn_readfirstlane(t_);
    copier.fetch([&](int s) __attribute__((always_inline)) -> int {
      const int i = 8 * (t - 1) + s;
      const int v = __builtin_amdgcn_readfirstlane(sgid[min(i, n_valid - 1)]);   // n_valid >= 1 here
      return i < n_valid ? v : 8 * J;
    });
  };
  // Tiles are copied in order: this wave's K blocks, then its V blocks; then the
  // next tile's groups are fetched.
  constexpr int BPW = GroupCopier<D, NW>::BPW;
  auto issue = [&](int t, auto B) __attribute__((always_inline)) {
    static_for<0, BPW>([&](auto K) { copier.template copy_one<K()>(KB(B), kb); });
    static_for<0, BPW>([&](auto K) { copier.template copy_one<K()>(VB(B), vb); });
    if (t + 1 < n_tiles) prepare(t + 1);
  };
  if (n_sel_tiles > 0) {   // the first selected tile travels while the own chunk is computed
    prepare(1);
    issue(1, ic<0>{});
  }

  RowOffsets<D> kro;      // K rows rho(n) (and 32 + rho(n): +32 rows as an immediate)
  kro.init(rho(n), h);
  ColOffsets<D> vco;      // V^T fragments
  vco.init(l);

  const float c2 = a.scale * kLog2e;
  float m2 = -INFINITY, lsum = 0.f;   // running maximum (log2 domain); this lane's share of the row sum
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  auto compute = [&](int t, auto B) __attribute__((always_inline)) {
    const uint16_t* K = KB(B);
    const uint16_t* V = VB(B);
    kro.refresh();
    vco.refresh();
    // S^T for 64 keys: two 32-key subtiles.  All K fragments are read in one batch,
    // then the MFMAs run (while copies into LDS are in flight the compiler can only
    // wait for all outstanding LDS reads at once).
    f32x16 s[2];
    {
      bf16x8 kfr[2][KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kfr[0][ks] = kro.read(K, ks);
        kfr[1][ks] = kro.template read<32 * D * 2>(K, ks);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[kt] = mfma32(kfr[kt][ks], qf[ks], s[kt]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
    }
    // Mask (only the own chunk and a partial last group tile need it), then the
    // online softmax in the log2 domain: max of the raw scores, scaled once
    // (scale > 0), and exp2(score * c2 - m) as one FMA per key.
    const bool local = t == 0;
    const bool full = !local && 8 * t <= n_valid;
    if (!full) {
      const int kv_lim = local ? pos : 8 * (n_valid - 8 * (t - 1)) - 1;   // last valid key index
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kt + out_row(r, h) > kv_lim) s[kt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = half_max(mx) * c2;   // finite: every row has a valid key in every tile
    // The running maximum only moves when a tile exceeds it by more than 2^8: P stays
    // below 256 and the rescale of O (64 multiplies) is skipped in almost every tile.
    // O and the normaliser share the maximum, so the result is unchanged.
    const bool grow = mx > m2 + 8.f;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mx : m2;
      const float alpha = fast_exp2(m2 - m_new);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m2 = m_new;
    }
    // P as bf16 operand fragments; the row sum adds the rounded values that the
    // P V product uses (two per v_dot2).
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(s[ks >> 1][8 * (ks & 1) + e], c2, -m2));
      pf[ks] = f32x8_to_bf16x8(pv);
      const uint4 u = __builtin_bit_cast(uint4, pf[ks]);
      lsum = add_bf16x2(u.x, lsum);
      lsum = add_bf16x2(u.y, lsum);
      lsum = add_bf16x2(u.z, lsum);
      lsum = add_bf16x2(u.w, lsum);
    }
    // O^T += V^T P^T over 4 k-steps of 16 keys (V^T fragments read as two batches).
    static_for<0, 2>([&](auto HALF) {
      bf16x8 vfr[2][DT];
      static_for<0, 2>([&](auto K2) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vfr[K2()][dt] = vco.template read<2 * HALF() + K2()>(V, dt);
      });
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32(vfr[k2][dt], pf[2 * HALF() + k2], oacc[dt]);
    });
  };

  // the own chunk (its copies were issued before the first selected tile's)
  if (n_sel_tiles > 0) wait_vmcnt<2 * BPW>(); else wait_vmcnt<0>();
  tile_barrier();
  compute(0, ic<2>{});
  // the selected tiles 1 .. n_sel_tiles through sets 0 and 1 (the first already issued)
  pipeline<2, 2 * BPW, /*PREISSUED=*/true>(
      n_sel_tiles, [&](int t, auto B) __attribute__((always_inline)) { issue(t + 1, B); },
      [&](int t, auto B) __attribute__((always_inline)) { compute(t + 1, B); });

  // Epilogue: lane holds row `pos`, columns 32dt + 8g + 4h + i (i = 0..3) for r = 4g + i.
  // O leaves through this wave's 32-row LDS region as whole rows; the barrier keeps
  // every region free until all waves have finished their last tile.
  const float ltot = half_sum(lsum);
  const float inv = 1.f / ltot;
  tile_barrier();
  store_rows32<D>(row_region(w), (uint16_t*)a.o + qrow0 * D, [&](int dt, int g) __attribute__((always_inline)) {
    return f32x4_to_bf16x4_bits(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                                oacc[dt][4 * g + 3] * inv);
  });
  if (h == 0) a.lse[qrow] = (m2 + log2f(ltot)) * kLn2;
}

// HPW query heads of the G sharing a KV head per work-group (2 waves of 32 rows each);
// the G / HPW work-groups of a unit gather the same tiles (the repeats hit L2: their
// ids are consecutive, hence on one XCD) but run unsynchronised, so one group's
// softmax overlaps another's MFMAs on the same CU.
template <int D, int G, int HPW>
__global__ __launch_bounds__(128 * HPW, 8 / (2 * HPW) > 1 ? 8 / (2 * HPW) : 1) void attend_fwd_bf16_kernel(FwdArgs a) {
  constexpr int KS = D / 16;       // k-steps over the head dimension
  // Tile buffer sets as distinct arrays: the compiler can then see that reads of one
  // never alias the asynchronous copies into another.
  __shared__ __align__(16) uint16_t k0[64 * D], v0[64 * D], k1[64 * D], v1[64 * D];
  __shared__ __align__(16) uint16_t k2[64 * D], v2[64 * D], k3[64 * D], v3[64 * D];
  __shared__ int sgid[512];
  auto KB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return k0; else if constexpr (B() == 1) return k1;
    else if constexpr (B() == 2) return k2; else return k3;
  };
  auto VB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return v0; else if constexpr (B() == 1) return v1;
    else if constexpr (B() == 2) return v2; else return v3;
  };

  const int item = xcd_unit(blockIdx.x, gridDim.x);
  if (item >= a.n_units * (G / HPW)) return;
  const int unit = item / (G / HPW);
  const int j = unit % a.nb;
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int w = threadIdx.x >> 6, h = (threadIdx.x & 63) >> 5, n = threadIdx.x & 31;
  const int hh = (item % (G / HPW)) * HPW + (w >> 1);   // query head within the KV group
  const int64_t qrow = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)j * kQBlock + 32 * (w & 1) + n;

  bf16x8 qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + qrow * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
  }

  // The group list (k_g <= 512) goes to LDS once; its valid entries (ascending, -1
  // only trails) are counted on the way.
  const int n_valid = __builtin_amdgcn_readfirstlane(
      count_valid<128 * HPW>(a.gidx + (int64_t)unit * a.kg, a.kg, sgid));   // ends with a barrier
  issue_own_tile<D, 2 * HPW>(a, unit, k2, v2);
  attend_unit_bf16<D, G, HPW>(a, unit, item % (G / HPW), qf, sgid, n_valid, KB, VB);
}

// Route, then attend, in one work-group per unit (4 query heads per KV head: 8
// waves).  The routing waves hold row tiles {w % 4, w % 4 + 4}; wave w attends with
// row tile w, one of the two, so the query rows are read once for both phases.  The
// summary batch buffers of the routing are the attention's tile buffer sets 0 and 1;
// the own chunk's tile is copied into set 2 once the chunk scores are in.  With LAG
// (strictly causal routing, ra.lag == 1) the block is routed by the rows of the block
// before it, and the attention then reads the block's own rows.
template <int D, bool LAG>
__global__ __launch_bounds__(512, 1) void route_attend_bf16_kernel(RouteArgs ra, FwdArgs a) {
  constexpr int G = 4;
  constexpr int KS = D / 16;
  __shared__ __align__(16) uint16_t k0[64 * D], v0[64 * D], k1[64 * D], v1[64 * D], k2[64 * D], v2[64 * D];
  __shared__ RouteShared<route_threads<G>()> sm;
  __shared__ int sgid[512];
  auto KB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return k0; else if constexpr (B() == 1) return k1; else return k2;
  };
  auto VB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return v0; else if constexpr (B() == 1) return v1; else return v2;
  };
  auto tile = [&](auto B, auto T) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (T() == 0) return KB(B); else return VB(B);
  };
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  bf16x8 qr[route_row_tiles_per_wave<G>()][KS];
  int nc, ng;
  // The own chunk's K / V travel while the chunks are selected and the groups scored.
  route_unit_bf16<D, G>(ra, unit, tile, sm, qr, nc, ng,
                        [&]() __attribute__((always_inline)) { issue_own_tile<D, 8>(a, unit, k2, v2); });
  // The selected groups as ids (ascending), for the tile copies.
  for (int i = tid; i < ng; i += 512) sgid[i] = 8 * sm.csel[sm.gsel[i] >> 3] + (sm.gsel[i] & 7);
  __syncthreads();
  bf16x8 qf[KS];
  if constexpr (LAG) {
    // row tile w of the block itself: query head w / 2 of the group, rows 32 (w % 2) ..
    const int l = tid & 63, h = l >> 5, n = l & 31;
    const int j = unit % a.nb, bh = unit / a.nb, b = bh / a.Hkv, kvh = bh % a.Hkv;
    const uint16_t* qp = (const uint16_t*)a.q +
        ((((int64_t)b * a.Hq + kvh * G + (w >> 1)) * a.seg_len) + (int64_t)j * kQBlock + 32 * (w & 1) + n) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = w < 4 ? qr[0][ks] : qr[1][ks];
  }
  attend_unit_bf16<D, G, G>(a, unit, 0, qf, sgid, __builtin_amdgcn_readfirstlane(ng), KB, VB);
}

// ---------------------------------------------------------------- fp32 (SIMT)
template <int D>
__global__ __launch_bounds__(512) void attend_fwd_f32_kernel(FwdArgs a, int G) {
  __shared__ int sgid[512];
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int j = unit % a.nb;
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int J = (int)(a.t_hist / kChunk) + j;
  const int nt = blockDim.x;
  int n_valid = 0;
  for (int i0 = 0; i0 < a.kg; i0 += nt) {
    const int i = i0 + threadIdx.x;
    int v = -1;
    if (i < a.kg) { v = a.gidx[(int64_t)unit * a.kg + i]; sgid[i] = v; }
    n_valid += __syncthreads_count(v >= 0);
  }
  const int hh = threadIdx.x / kQBlock, pos = threadIdx.x % kQBlock;
  const int64_t qrow = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)j * kQBlock + pos;
  const float* qp = (const float*)a.q + qrow * D;
  const float* kb = (const float*)a.k + (int64_t)bh * a.t_cap * D;
  const float* vb = (const float*)a.v + (int64_t)bh * a.t_cap * D;
  float qv[D], acc[D];
  for (int e = 0; e < D; ++e) { qv[e] = qp[e]; acc[e] = 0.f; }
  float m = -INFINITY, lsum = 0.f;
  const int n_keys = 8 * n_valid + pos + 1;
  for (int i = 0; i < n_keys; ++i) {
    const int64_t tok = i < 8 * n_valid ? (int64_t)kGroup * sgid[i >> 3] + (i & 7)
                                        : (int64_t)kChunk * J + (i - 8 * n_valid);
    const float* kr = kb + tok * D;
    float dot = 0.f;
    for (int e = 0; e < D; ++e) dot = fmaf(qv[e], kr[e], dot);
    const float x = dot * a.scale;
    const float m_new = fmaxf(m, x);
    const float alpha = expf(m - m_new);
    const float p = expf(x - m_new);
    lsum = lsum * alpha + p;
    const float* vr = vb + tok * D;
    for (int e = 0; e < D; ++e) acc[e] = acc[e] * alpha + p * vr[e];
    m = m_new;
  }
  float* op = (float*)a.o + qrow * D;
  for (int e = 0; e < D; ++e) op[e] = acc[e] / lsum;
  a.lse[qrow] = m + logf(lsum);
}

template <int D, int G>
hipError_t launch_bf16(const FwdArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  constexpr int HPW = G >= 8 ? 4 : G;   // query heads per work-group
  return launch_kernel_timed(attend_fwd_bf16_kernel<D, G, HPW>, dim3(xcd_grid(a.n_units * (G / HPW))),
                             dim3(128 * HPW), s, start, stop, a);
}
template <int D>
hipError_t launch_bf16_g(const FwdArgs& a, int G, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  switch (G) {
    case 1: return launch_bf16<D, 1>(a, s, start, stop);
    case 2: return launch_bf16<D, 2>(a, s, start, stop);
    case 4: return launch_bf16<D, 4>(a, s, start, stop);
    default: return launch_bf16<D, 8>(a, s, start, stop);
  }
}

FwdArgs fwd_args(const Dims& d, const void* q, const void* k, const void* v, const int32_t* group_idx, void* o,
                 float* lse) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.gidx = group_idx; a.o = o; a.lse = lse;
  a.t_cap = d.t_cap; a.t_hist = d.t_hist; a.seg_len = d.seg_len;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kg = d.kg; a.nb = d.nb; a.n_units = d.B * d.Hkv * d.nb;
  a.scale = d.scale;
  return a;
}

}  // namespace

hipError_t launch_attend_fwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const int32_t* group_idx, void* o, float* lse, hipStream_t s, hipEvent_t start,
                             hipEvent_t stop) {
  const FwdArgs a = fwd_args(d, q, k, v, group_idx, o, lse);
  const int grid = xcd_grid(a.n_units);
  if (bf16) return d.D == 128 ? launch_bf16_g<128>(a, d.G, s, start, stop) : launch_bf16_g<64>(a, d.G, s, start, stop);
  return d.D == 128
             ? launch_kernel_timed(attend_fwd_f32_kernel<128>, dim3(grid), dim3(64 * d.G), s, start, stop, a, d.G)
             : launch_kernel_timed(attend_fwd_f32_kernel<64>, dim3(grid), dim3(64 * d.G), s, start, stop, a, d.G);
}

hipError_t launch_forward(const Dims& d, bool bf16, const void* q, const void* q_prev, bool causal, const void* k,
                          const void* v, void* chunk_sum, void* group_sum, int32_t* chunk_idx, int32_t* group_idx,
                          void* o, float* lse, hipStream_t s, const hipEvent_t* ev) {
  const hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  const hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
  hipError_t e = launch_summaries(d, bf16, k, d.t_hist, d.t_hist + d.seg_len, group_sum, chunk_sum, s, e0, e1);
  if (e != hipSuccess) return e;
  if (!(bf16 && d.G == 4)) {
    e = launch_route(d, bf16, q, q_prev, causal, chunk_sum, group_sum, chunk_idx, group_idx, nullptr, nullptr, s,
                     e2, nullptr);
    if (e != hipSuccess) return e;
    return launch_attend_fwd(d, bf16, q, k, v, group_idx, o, lse, s, nullptr, e3);
  }
  RouteArgs ra;
  ra.q = q; ra.q_prev = q_prev; ra.lag = causal ? 1 : 0;
  ra.csum = chunk_sum; ra.gsum = group_sum;
  ra.cidx = chunk_idx; ra.gidx = group_idx; ra.cscore = nullptr; ra.gscore = nullptr;
  ra.t_cap = d.t_cap; ra.t_hist = d.t_hist; ra.seg_len = d.seg_len;
  ra.Hq = d.Hq; ra.Hkv = d.Hkv; ra.kc = d.kc; ra.kg = d.kg; ra.nb = d.nb;
  ra.n_units = d.B * d.Hkv * d.nb;
  const FwdArgs a = fwd_args(d, q, k, v, group_idx, o, lse);
  const dim3 grid(xcd_grid(a.n_units));
  if (causal)
    return d.D == 128 ? launch_kernel_timed(route_attend_bf16_kernel<128, true>, grid, dim3(512), s, e2, e3, ra, a)
                      : launch_kernel_timed(route_attend_bf16_kernel<64, true>, grid, dim3(512), s, e2, e3, ra, a);
  return d.D == 128 ? launch_kernel_timed(route_attend_bf16_kernel<128, false>, grid, dim3(512), s, e2, e3, ra, a)
                    : launch_kernel_timed(route_attend_bf16_kernel<64, false>, grid, dim3(512), s, e2, e3, ra, a);
}

}  // namespace hga
