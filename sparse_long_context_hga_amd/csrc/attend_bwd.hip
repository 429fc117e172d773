// Backward of the routed attention for the active segment only.
//
// Pages: adnankhan.ai note "Long-Context Fine-Tuning with Limited VRAM", section
// "Raw Abstract / Excerpt" (only the active segment stays differentiable; older
// K/V is detached) and seventnews "BMW如何通过重新设计注意力机制，在16 GB GPU上实现16K上下文",
// section "HGA的不同之处" (segment-wise backprop; the router has no weights, so
// gradients reach only the exact-token attention).  Softmax-attention gradient:
//   D = rowsum(dO * O),  P = exp(scale q.k - LSE),  dP = dO . v,  dS = P (dP - D)
//   dQ = scale sum_t dS k_t;   for active t:  dV_t = sum P dO,  dK_t = scale sum dS q
// History tokens (< t_hist) receive nothing.
//
// Two kernels, both deterministic (no floating-point atomics):
//  * dq  (query-major, one work-group per (sequence, KV head, query block)):
//    same gathered tiles as the forward; recomputes P from LSE; writes dQ and
//    D = rowsum(dO * O) (workspace) for the second kernel;
//  * dkdv (key-major, one work-group per (sequence, KV head, active chunk)): the
//    chunk's 64 keys stay in registers; it visits its own block (causal) and
//    every later block whose selection contains one of its groups, staging that
//    block's Q / dO rows per query head in swizzled LDS, and accumulates dK, dV
//    in fp32 registers (dV^T += dO^T P, dK^T += Q^T dS, with the transposing
//    LDS reads supplying the k-contiguous operands).
#include "hga_device.h"
#include "hga_internal.h"

#include <math.h>

namespace hga {
namespace {

constexpr int kMaxBlocks = 1024;   // query blocks per segment supported by the dkdv kernel

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;
  const int32_t* gidx;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;      // [B, Hq, S] rowsum(dO * O)
  int64_t t_cap, t_hist, seg_len;
  int Hq, Hkv, kg, nb, n_units;
  float scale;
};

__device__ __forceinline__ float dot8_bf16(bf16x8 x, bf16x8 y) {
  const uint4 a = __builtin_bit_cast(uint4, x), b = __builtin_bit_cast(uint4, y);
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __uint_as_float(av[i] << 16) * __uint_as_float(bv[i] << 16);
    s += __uint_as_float(av[i] & 0xFFFF0000u) * __uint_as_float(bv[i] & 0xFFFF0000u);
  }
  return s;
}

// ---------------------------------------------------------------- dQ (bf16)
template <int D, int G>
__global__ __launch_bounds__(128 * G) void attend_bwd_dq_bf16_kernel(BwdArgs a) {
  constexpr int NT = 128 * G;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  __shared__ __align__(16) uint16_t tk[2][64 * D];
  __shared__ __align__(16) uint16_t tv[2][64 * D];
  __shared__ int sgid[512];

  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int j = unit % a.nb;
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = l & 31;
  const int hh = w >> 1;
  const int pos = 32 * (w & 1) + n;
  const int64_t qrow = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)j * kQBlock + pos;
  const uint16_t* kb = (const uint16_t*)a.k + (int64_t)bh * a.t_cap * D;
  const uint16_t* vb = (const uint16_t*)a.v + (int64_t)bh * a.t_cap * D;

  bf16x8 qf[KS], dof[KS];
  float dpart = 0.f;
  {
    const uint16_t* qp = (const uint16_t*)a.q + qrow * D;
    const uint16_t* dp = (const uint16_t*)a.d_o + qrow * D;
    const uint16_t* op = (const uint16_t*)a.o + qrow * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * h);
      dof[ks] = *reinterpret_cast<const bf16x8*>(dp + 16 * ks + 8 * h);
      dpart += dot8_bf16(dof[ks], *reinterpret_cast<const bf16x8*>(op + 16 * ks + 8 * h));
    }
  }
  const float Dr = wave_sum32(dpart);
  if (h == 0) a.dvec[qrow] = Dr;
  const float lse2 = a.lse[qrow] * kLog2e;

  const int n_valid = count_valid<NT>(a.gidx + (int64_t)unit * a.kg, a.kg, sgid);
  const int n_sel_tiles = (n_valid + 7) >> 3;
  const int n_tiles = n_sel_tiles + 1;
  TileLoader<D, NT> ld;
  ld.load(kb, vb, 0, n_sel_tiles, n_valid, sgid, J);
  ld.store(tk[0], tv[0]);

  const float c2 = a.scale * kLog2e;
  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = f32x16{};

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) ld.load(kb, vb, t + 1, n_sel_tiles, n_valid, sgid, J);
    __syncthreads();
    const uint16_t* K = tk[buf];
    const uint16_t* V = tv[buf];
    const bool local = t == n_sel_tiles;
    const int kv_lim = local ? pos : 8 * (n_valid - 8 * t) - 1;
    // One 32-key subtile at a time keeps the live score registers to 2 x 16.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 s = {}, dpv = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(lds_row8<D>(K, 32 * kt + rho(n), 16 * ks + 8 * h), qf[ks], s);
        dpv = mfma32(lds_row8<D>(V, 32 * kt + rho(n), 16 * ks + 8 * h), dof[ks], dpv);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + out_row(r, h);
        const float p = key <= kv_lim ? exp2f(s[r] * c2 - lse2) : 0.f;
        ds[r] = p * (dpv[r] - Dr);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 dsf = f32x8_to_bf16x8(ds + 8 * half);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          dqacc[dt] = mfma32(lds_col8<D>(K, 32 * kt + 16 * half, 32 * dt), dsf, dqacc[dt]);
      }
    }
    if (t + 1 < n_tiles) ld.store(tk[buf ^ 1], tv[buf ^ 1]);
  }

  uint16_t* qo = (uint16_t*)a.dq + qrow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * dt + 8 * g + 4 * h;
      *reinterpret_cast<uint2*>(qo + col) =
          make_uint2(pack_bf16x2(dqacc[dt][4 * g] * a.scale, dqacc[dt][4 * g + 1] * a.scale),
                     pack_bf16x2(dqacc[dt][4 * g + 2] * a.scale, dqacc[dt][4 * g + 3] * a.scale));
    }
}

// ---------------------------------------------------------------- dK/dV (bf16)
// 4 waves: wave w owns keys 32*(w&1) .. +31 of the chunk and, for every staged
// 64-row tile, the rows 32*(w>>1) .. +31; the two row halves are summed at the end.
template <int D, int G>
__global__ __launch_bounds__(256) void attend_bwd_dkdv_bf16_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CH = D / 8;
  __shared__ __align__(16) uint16_t tqdo[2 * 64 * D];   // Q tile, then dO tile
  __shared__ float slse[64], sdr[64];
  __shared__ uint32_t vmask[kMaxBlocks];
  uint16_t* tq = tqdo;
  uint16_t* tdo = tqdo + 64 * D;

  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int cc = unit % a.nb;                      // active chunk == its own query block
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int64_t cglob = a.t_hist / kChunk + cc;    // global chunk id
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = l & 31;
  const int kh = w & 1, rh = w >> 1;
  const int key = 32 * kh + n;                     // this lane's key (operand-B column)
  const int64_t tok = cglob * kChunk + key;

  bf16x8 kf[KS], vf[KS];
  {
    const uint16_t* kp = (const uint16_t*)a.k + ((int64_t)bh * a.t_cap + tok) * D;
    const uint16_t* vp = (const uint16_t*)a.v + ((int64_t)bh * a.t_cap + tok) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(kp + 16 * ks + 8 * h);
      vf[ks] = *reinterpret_cast<const bf16x8*>(vp + 16 * ks + 8 * h);
    }
  }

  // Which later blocks selected groups of this chunk (bit u = group 8*cglob + u).
  for (int i = tid; i < a.nb; i += 256) vmask[i] = 0u;
  __syncthreads();
  for (int jj = cc + 1 + w; jj < a.nb; jj += 4) {
    const int32_t* g = a.gidx + ((int64_t)bh * a.nb + jj) * a.kg;
    for (int i = l; i < a.kg; i += 64) {
      const int64_t gid = g[i];
      if (gid >= cglob * 8 && gid < cglob * 8 + 8) atomicOr(&vmask[jj], 1u << (int)(gid - cglob * 8));
    }
  }
  __syncthreads();

  const float c2 = a.scale * kLog2e;
  f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) { dvacc[dt] = f32x16{}; dkacc[dt] = f32x16{}; }

  for (int jj = cc; jj < a.nb; ++jj) {
    const uint32_t mask = jj == cc ? 0xFFu : vmask[jj];
    if (mask == 0u) continue;
    for (int hh = 0; hh < G; ++hh) {
      const int64_t qrow0 = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)jj * kQBlock;
      const uint16_t* qp = (const uint16_t*)a.q + qrow0 * D;
      const uint16_t* dp = (const uint16_t*)a.d_o + qrow0 * D;
      for (int idx = tid; idx < 64 * CH; idx += 256) {
        const int r = idx / CH, c = idx % CH;
        const int off = r * D + 8 * swz_chunk<D>(r, c);
        *reinterpret_cast<uint4*>(tq + off) = *reinterpret_cast<const uint4*>(qp + (int64_t)r * D + 8 * c);
        *reinterpret_cast<uint4*>(tdo + off) = *reinterpret_cast<const uint4*>(dp + (int64_t)r * D + 8 * c);
      }
      if (tid < 64) {
        slse[tid] = a.lse[qrow0 + tid] * kLog2e;
        sdr[tid] = a.dvec[qrow0 + tid];
      }
      __syncthreads();

      f32x16 s = {}, dpv = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(lds_row8<D>(tq, 32 * rh + rho(n), 16 * ks + 8 * h), kf[ks], s);
        dpv = mfma32(lds_row8<D>(tdo, 32 * rh + rho(n), 16 * ks + 8 * h), vf[ks], dpv);
      }
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rh + out_row(r, h);
        const bool valid = jj == cc ? key <= row : ((mask >> (key >> 3)) & 1u) != 0u;
        p[r] = valid ? exp2f(s[r] * c2 - slse[row]) : 0.f;
        ds[r] = p[r] * (dpv[r] - sdr[row]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pf = f32x8_to_bf16x8(p + 8 * ks);
        const bf16x8 dsf = f32x8_to_bf16x8(ds + 8 * ks);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dvacc[dt] = mfma32(lds_col8<D>(tdo, 32 * rh + 16 * ks, 32 * dt), pf, dvacc[dt]);
          dkacc[dt] = mfma32(lds_col8<D>(tq, 32 * rh + 16 * ks, 32 * dt), dsf, dkacc[dt]);
        }
      }
      __syncthreads();
    }
  }

  // Sum the two row halves (waves 2,3 -> waves 0,1) through LDS, one tensor at a time.
  float* red = reinterpret_cast<float*>(tqdo);   // 2 * 64 * D bf16 = room for 2 * DT * 16 * 64 floats
  const int64_t orow = (int64_t)bh * a.seg_len + (int64_t)cc * kChunk + key;
  auto reduce_store = [&](f32x16 (&acc)[DT], void* dst, float sc) {
    if (rh == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((kh * DT + dt) * 16 + r) * 64 + l] = acc[dt][r];
    }
    __syncthreads();
    if (rh == 0) {
      uint16_t* out = (uint16_t*)dst + orow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = (acc[dt][4 * g + i] + red[((kh * DT + dt) * 16 + 4 * g + i) * 64 + l]) * sc;
          const int col = 32 * dt + 8 * g + 4 * h;
          *reinterpret_cast<uint2*>(out + col) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
        }
    }
    __syncthreads();
  };
  reduce_store(dvacc, a.dv, 1.f);
  reduce_store(dkacc, a.dk, a.scale);
}

// ---------------------------------------------------------------- fp32 (SIMT)
template <int D>
__global__ __launch_bounds__(512) void attend_bwd_dq_f32_kernel(BwdArgs a, int G) {
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
  const float* dop = (const float*)a.d_o + qrow * D;
  const float* op = (const float*)a.o + qrow * D;
  const float* kb = (const float*)a.k + (int64_t)bh * a.t_cap * D;
  const float* vb = (const float*)a.v + (int64_t)bh * a.t_cap * D;
  float qv[D], dov[D], dq[D];
  float Dr = 0.f;
  for (int e = 0; e < D; ++e) { qv[e] = qp[e]; dov[e] = dop[e]; dq[e] = 0.f; Dr = fmaf(dov[e], op[e], Dr); }
  a.dvec[qrow] = Dr;
  const float lse = a.lse[qrow];
  const int n_keys = 8 * n_valid + pos + 1;
  for (int i = 0; i < n_keys; ++i) {
    const int64_t tok = i < 8 * n_valid ? (int64_t)kGroup * sgid[i >> 3] + (i & 7)
                                        : (int64_t)kChunk * J + (i - 8 * n_valid);
    const float* kr = kb + tok * D;
    const float* vr = vb + tok * D;
    float s = 0.f, dp = 0.f;
    for (int e = 0; e < D; ++e) { s = fmaf(qv[e], kr[e], s); dp = fmaf(dov[e], vr[e], dp); }
    const float p = expf(s * a.scale - lse);
    const float ds = p * (dp - Dr);
    for (int e = 0; e < D; ++e) dq[e] = fmaf(ds, kr[e], dq[e]);
  }
  float* out = (float*)a.dq + qrow * D;
  for (int e = 0; e < D; ++e) out[e] = dq[e] * a.scale;
}

// 256 threads = 64 keys x 4 column quarters.
template <int D>
__global__ __launch_bounds__(256) void attend_bwd_dkdv_f32_kernel(BwdArgs a, int G) {
  constexpr int DQ = D / 4;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  if (unit >= a.n_units) return;
  const int cc = unit % a.nb;
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int64_t cglob = a.t_hist / kChunk + cc;
  const int key = threadIdx.x >> 2, qt = threadIdx.x & 3;
  const int64_t tok = cglob * kChunk + key;
  const float* kp = (const float*)a.k + ((int64_t)bh * a.t_cap + tok) * D + qt * DQ;
  const float* vp = (const float*)a.v + ((int64_t)bh * a.t_cap + tok) * D + qt * DQ;
  float kq[DQ], vq[DQ], dk[DQ], dv[DQ];
  for (int e = 0; e < DQ; ++e) { kq[e] = kp[e]; vq[e] = vp[e]; dk[e] = 0.f; dv[e] = 0.f; }
  for (int jj = cc; jj < a.nb; ++jj) {
    bool attends = jj == cc;
    if (!attends) {
      const int32_t* g = a.gidx + ((int64_t)bh * a.nb + jj) * a.kg;
      for (int i = 0; i < a.kg; ++i) attends |= g[i] == (int32_t)(tok / kGroup);
    }
    // Every lane of a 4-lane key group shares `attends`; lanes of different keys may
    // differ, so all lanes walk the rows and mask (the shuffles need every lane).
    for (int hh = 0; hh < G; ++hh)
      for (int pos = 0; pos < kQBlock; ++pos) {
        const int64_t qrow = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)jj * kQBlock + pos;
        const float* qr = (const float*)a.q + qrow * D + qt * DQ;
        const float* dor = (const float*)a.d_o + qrow * D + qt * DQ;
        float s = 0.f, dp = 0.f;
        for (int e = 0; e < DQ; ++e) { s = fmaf(qr[e], kq[e], s); dp = fmaf(dor[e], vq[e], dp); }
        s += __shfl_xor(s, 1, 64); s += __shfl_xor(s, 2, 64);
        dp += __shfl_xor(dp, 1, 64); dp += __shfl_xor(dp, 2, 64);
        const bool valid = jj == cc ? key <= pos : attends;
        const float p = valid ? expf(s * a.scale - a.lse[qrow]) : 0.f;
        const float ds = p * (dp - a.dvec[qrow]);
        for (int e = 0; e < DQ; ++e) { dv[e] = fmaf(p, dor[e], dv[e]); dk[e] = fmaf(ds, qr[e], dk[e]); }
      }
  }
  const int64_t orow = (int64_t)bh * a.seg_len + (int64_t)cc * kChunk + key;
  float* dko = (float*)a.dk + orow * D + qt * DQ;
  float* dvo = (float*)a.dv + orow * D + qt * DQ;
  for (int e = 0; e < DQ; ++e) { dko[e] = dk[e] * a.scale; dvo[e] = dv[e]; }
}

template <int D, int G>
void launch_bf16(const BwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attend_bwd_dq_bf16_kernel<D, G>), dim3(grid), dim3(128 * G), 0, s, a);
  hipLaunchKernelGGL((attend_bwd_dkdv_bf16_kernel<D, G>), dim3(grid), dim3(256), 0, s, a);
}
template <int D>
void launch_bf16_g(const BwdArgs& a, int G, int grid, hipStream_t s) {
  switch (G) {
    case 1: launch_bf16<D, 1>(a, grid, s); break;
    case 2: launch_bf16<D, 2>(a, grid, s); break;
    case 4: launch_bf16<D, 4>(a, grid, s); break;
    default: launch_bf16<D, 8>(a, grid, s); break;
  }
}

}  // namespace

size_t bwd_workspace_bytes(const Dims& d) {
  const size_t rows = (size_t)d.B * d.Hq * (size_t)d.seg_len;
  return ((rows * sizeof(float)) + 255) & ~(size_t)255;
}

hipError_t launch_attend_bwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* d_o,
                             const int32_t* group_idx, void* dq, void* dk, void* dv,
                             void* workspace, hipStream_t s) {
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.d_o = d_o; a.lse = lse; a.gidx = group_idx;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dvec = (float*)workspace;
  a.t_cap = d.t_cap; a.t_hist = d.t_hist; a.seg_len = d.seg_len;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kg = d.kg; a.nb = d.nb; a.n_units = d.B * d.Hkv * d.nb;
  a.scale = d.scale;
  const int grid = xcd_grid(a.n_units);
  if (bf16) {
    if (d.D == 128) launch_bf16_g<128>(a, d.G, grid, s);
    else launch_bf16_g<64>(a, d.G, grid, s);
  } else {
    if (d.D == 128) {
      hipLaunchKernelGGL((attend_bwd_dq_f32_kernel<128>), dim3(grid), dim3(64 * d.G), 0, s, a, d.G);
      hipLaunchKernelGGL((attend_bwd_dkdv_f32_kernel<128>), dim3(grid), dim3(256), 0, s, a, d.G);
    } else {
      hipLaunchKernelGGL((attend_bwd_dq_f32_kernel<64>), dim3(grid), dim3(64 * d.G), 0, s, a, d.G);
      hipLaunchKernelGGL((attend_bwd_dkdv_f32_kernel<64>), dim3(grid), dim3(256), 0, s, a, d.G);
    }
  }
  return hipGetLastError();
}

}  // namespace hga
