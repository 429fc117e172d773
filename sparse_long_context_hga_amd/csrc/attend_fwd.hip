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
//   * key tiles of 64 tokens = 8 selected groups (each group is one contiguous
//     2 KiB run of K and of V in HBM), then the own chunk; two buffer sets in
//     swizzled LDS, the next tile's copies in flight during the MFMAs;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys in rho order, B = the
//     wave's 32 query rows held in registers): each lane ends with one query row
//     and 32 of the 64 keys, so the online-softmax statistics live in the lane;
//   * O^T += V^T P^T: P (bf16) is already in operand-B layout thanks to rho, and
//     V^T comes from the row-major tile through ds_read_b64_tr_b16.
// fp32 path: one thread per query row, plain fp32 loops (exact-precision mode).
#include "hga_device.h"
#include "hga_internal.h"

#include <math.h>

namespace hga {
namespace {

constexpr int kStages = 2;   // K/V tile buffer sets (tiles in flight + 1); two measured 2% faster than three

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

// HPW query heads of the G sharing a KV head per work-group (2 waves of 32 rows each);
// the G / HPW work-groups of a unit gather the same tiles (the repeats hit L2: their
// ids are consecutive, hence on one XCD) but run unsynchronised, so one group's
// softmax overlaps another's MFMAs on the same CU.
template <int D, int G, int HPW>
__global__ __launch_bounds__(128 * HPW, 8 / (2 * HPW) > 1 ? 8 / (2 * HPW) : 1) void attend_fwd_bf16_kernel(FwdArgs a) {
  constexpr int NW = 2 * HPW;
  constexpr int kStagesHere = HPW == G ? kStages : 2;
  constexpr int KS = D / 16;       // k-steps over the head dimension
  constexpr int DT = D / 32;       // 32-wide column tiles of O^T
  // Tile buffer sets as distinct arrays: the compiler can then see that reads of one
  // never alias the asynchronous copies into another.
  __shared__ __align__(16) uint16_t k0[64 * D], v0[64 * D], k1[64 * D], v1[64 * D];
  __shared__ __align__(16) uint16_t k2[64 * D], v2[64 * D], k3[64 * D], v3[64 * D];
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
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = l & 31;
  const int hh = (item % (G / HPW)) * HPW + (w >> 1);   // query head within the KV group
  const int pos = 32 * (w & 1) + n;       // this lane's query position in the block
  // First row of this wave's 32 (wave-uniform) and this lane's row.
  const int64_t qrow0 = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)j * kQBlock + 32 * (w & 1);
  const int64_t qrow = qrow0 + n;

  const char* kb = (const char*)a.k + (int64_t)bh * a.t_cap * D * 2;
  const char* vb = (const char*)a.v + (int64_t)bh * a.t_cap * D * 2;
  // 32-row LDS region of wave wv in the first two tile buffer sets (for O after the
  // last tile).
  auto row_region = [&](int wv) __attribute__((always_inline)) -> uint16_t* {
    uint16_t* base = (wv >> 1) == 0 ? k0 : (wv >> 1) == 1 ? v0 : (wv >> 1) == 2 ? k1 : v1;
    return base + (wv & 1) * 32 * D;
  };

  bf16x8 qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + qrow * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
  }

  // The group list (k_g <= 512) goes to LDS once; its valid entries (ascending, -1
  // only trails) are counted on the way.
  __shared__ int sgid[512];
  const int n_valid = __builtin_amdgcn_readfirstlane(
      count_valid<128 * HPW>(a.gidx + (int64_t)unit * a.kg, a.kg, sgid));   // ends with a barrier
  const int n_sel_tiles = (n_valid + 7) >> 3;
  const int n_tiles = n_sel_tiles + 1;

  // Group of slot s (0..7) of tile t (wave-uniform): the selection, then the own
  // chunk as the last tile.  Slots past the selection repeat the own chunk's first
  // group (masked later).
  GroupCopier<D, NW> copier;
  auto prepare = [&](int t_) __attribute__((always_inline)) {
    const int t = __builtin_amdgcn_readfirstlane(t_);
    copier.fetch([&](int s) __attribute__((always_inline)) -> int {
      if (t < n_sel_tiles) {
        const int i = 8 * t + s;
        const int v = __builtin_amdgcn_readfirstlane(sgid[min(i, n_valid - 1)]);   // n_valid >= 1 here
        return i < n_valid ? v : 8 * J;
      }
      return 8 * J + s;
    });
  };
  // Tiles are copied in order 0, 1, 2, ...: this wave's K blocks, then its V blocks;
  // then the next tile's groups are fetched.
  constexpr int BPW = GroupCopier<D, NW>::BPW;
  auto issue = [&](int t, auto B) __attribute__((always_inline)) {
    static_for<0, BPW>([&](auto K) { copier.template copy_one<K()>(KB(B), kb); });
    static_for<0, BPW>([&](auto K) { copier.template copy_one<K()>(VB(B), vb); });
    if (t + 1 < n_tiles) prepare(t + 1);
  };
  prepare(0);

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
    const bool local = t == n_sel_tiles;
    const bool full = !local && 8 * (t + 1) <= n_valid;
    if (!full) {
      const int kv_lim = local ? pos : 8 * (n_valid - 8 * t) - 1;   // last valid key index
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

  pipeline<kStagesHere, 2 * BPW>(n_tiles, issue, compute);

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
hipError_t launch_bf16(const FwdArgs& a, hipStream_t s) {
  constexpr int HPW = G >= 8 ? 4 : G;   // query heads per work-group
  return launch_kernel(attend_fwd_bf16_kernel<D, G, HPW>, dim3(xcd_grid(a.n_units * (G / HPW))), dim3(128 * HPW),
                       s, a);
}
template <int D>
hipError_t launch_bf16_g(const FwdArgs& a, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_bf16<D, 1>(a, s);
    case 2: return launch_bf16<D, 2>(a, s);
    case 4: return launch_bf16<D, 4>(a, s);
    default: return launch_bf16<D, 8>(a, s);
  }
}

}  // namespace

hipError_t launch_attend_fwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const int32_t* group_idx, void* o, float* lse, hipStream_t s) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.gidx = group_idx; a.o = o; a.lse = lse;
  a.t_cap = d.t_cap; a.t_hist = d.t_hist; a.seg_len = d.seg_len;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kg = d.kg; a.nb = d.nb; a.n_units = d.B * d.Hkv * d.nb;
  a.scale = d.scale;
  const int grid = xcd_grid(a.n_units);
  if (bf16) return d.D == 128 ? launch_bf16_g<128>(a, d.G, s) : launch_bf16_g<64>(a, d.G, s);
  return d.D == 128 ? launch_kernel(attend_fwd_f32_kernel<128>, dim3(grid), dim3(64 * d.G), s, a, d.G)
                    : launch_kernel(attend_fwd_f32_kernel<64>, dim3(grid), dim3(64 * d.G), s, a, d.G);
}

}  // namespace hga
