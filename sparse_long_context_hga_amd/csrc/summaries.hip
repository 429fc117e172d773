// Group and chunk summaries of the keys (mean of 8 / 64 keys).
//
// Pages: the seventnews article "BMW如何通过重新设计注意力机制，在16 GB GPU上实现16K上下文",
// section "HGA的不同之处" (a compact summary vector per 64-token chunk, 8-token
// groups inside), and the gist.science summary, section "解决方案" (summary cards
// per chunk, a summary cache for the groups).  The formula is this library's
// definition: mean of the keys in the fixed fp32 pairwise order
//   group sum = ((k0+k1)+(k2+k3)) + ((k4+k5)+(k6+k7)),  chunk sum = same tree over
//   the 8 unscaled group sums;  stored as sum/8 and sum/64 in the key dtype.
//
// HBM-bound stream: one work-group per (chunk, KV head, sequence) reads the
// chunk's 64 keys once (coalesced rows) and writes 8 group rows and 1 chunk row.
#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ void load4(const float* p, float* x) {
    float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static __device__ __forceinline__ float cast(float x) { return x; }
  static __device__ __forceinline__ void store4(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
  static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ void load4(const uint16_t* p, float* x) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xFFFF0000u);
    x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
  static __device__ __forceinline__ void store4(uint16_t* p, const float* x) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
  static __device__ __forceinline__ void store1(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

__device__ __forceinline__ float tree8(const float* x) {
  const float a = (x[0] + x[1]) + (x[2] + x[3]);
  const float b = (x[4] + x[5]) + (x[6] + x[7]);
  return a + b;
}

// grid (chunks in range, Hkv, B); block = 8 groups x D/4 threads.
template <typename T, int D>
__global__ __launch_bounds__(2 * D) void summaries_kernel(const T* __restrict__ k, int64_t t_cap,
                                                          int64_t c_begin, T* __restrict__ gsum,
                                                          T* __restrict__ csum) {
  constexpr int TPG = D / 4;  // threads per group, 4 columns each
  __shared__ float gs_sh[8][D];
  const int tid = threadIdx.x;
  const int g = tid / TPG, cq = tid % TPG;
  const int64_t c = c_begin + blockIdx.x;
  const int64_t bh = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const T* kp = k + (bh * t_cap + c * kChunk + g * kGroup) * D + cq * 4;

  float x[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) Elem<T>::load4(kp + (int64_t)r * D, x[r]);
  float s[4], mean[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float col[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) col[r] = x[r][e];
    s[e] = tree8(col);
    mean[e] = s[e] * 0.125f;
    gs_sh[g][cq * 4 + e] = s[e];
  }
  Elem<T>::store4(gsum + (bh * (t_cap / kGroup) + c * 8 + g) * D + cq * 4, mean);
  __syncthreads();
  if (tid < D) {
    float col[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) col[u] = gs_sh[u][tid];
    Elem<T>::store1(csum + (bh * (t_cap / kChunk) + c) * D + tid, tree8(col) * 0.015625f);
  }
}

template <typename T, int D>
hipError_t launch_t(const Dims& d, const void* k, int64_t t_begin, int64_t t_end, void* gs, void* cs,
                    hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const int64_t nch = (t_end - t_begin) / kChunk;
  if (nch == 0) return hipSuccess;
  dim3 grid((unsigned)nch, (unsigned)d.Hkv, (unsigned)d.B);
  return launch_kernel_timed(summaries_kernel<T, D>, grid, dim3(2 * D), s, start, stop, (const T*)k, d.t_cap,
                             t_begin / kChunk, (T*)gs, (T*)cs);
}

}  // namespace

hipError_t launch_summaries(const Dims& d, bool bf16, const void* k, int64_t t_begin, int64_t t_end,
                            void* gs, void* cs, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (bf16) {
    return d.D == 128 ? launch_t<uint16_t, 128>(d, k, t_begin, t_end, gs, cs, s, start, stop)
                      : launch_t<uint16_t, 64>(d, k, t_begin, t_end, gs, cs, s, start, stop);
  }
  return d.D == 128 ? launch_t<float, 128>(d, k, t_begin, t_end, gs, cs, s, start, stop)
                    : launch_t<float, 64>(d, k, t_begin, t_end, gs, cs, s, start, stop);
}

}  // namespace hga
