// Device-side helpers shared by the HGA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kChunk = 64;    // tokens per chunk
constexpr int kGroup = 8;     // tokens per group
constexpr int kQBlock = 64;   // query positions per routing block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__device__ __forceinline__ bf16x8 f32x8_to_bf16x8(const float* x) {
  uint4 u;
  u.x = pack_bf16x2(x[0], x[1]);
  u.y = pack_bf16x2(x[2], x[3]);
  u.z = pack_bf16x2(x[4], x[5]);
  u.w = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// ------------------------------------------------------- orderable score keys
// Monotone map float -> uint32 (larger float -> larger key); -0 and +0 share a key.
// Every finite score maps above 0, so 0 marks "no score yet".
__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------ unit placement
// Work-groups are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// Launch 8*ceil(n/8) blocks and renumber so that consecutive unit ids (which
// share a sequence and KV head, hence K/V and summaries) land on one XCD's L2.
__device__ __forceinline__ int xcd_unit(int block, int n_launched) {
  const int per = n_launched >> 3;
  return (block & 7) * per + (block >> 3);
}
static inline int xcd_grid(int n_units) { return ((n_units + 7) / 8) * 8; }

// ------------------------------------------------------------ block scan
// Exclusive prefix sum of one int per thread over a block of NT threads
// (NT a multiple of 64, at most 1024).  `sh` holds NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int t = sh[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// ------------------------------------------------------------ LDS tiles
// A tile is 64 rows x D bf16, row-major, with the 16-byte chunks of each row
// permuted by an XOR swizzle so that both access patterns of the kernels are
// free of bank conflicts: 16 lanes reading 16 B from 16 consecutive rows, and
// the transposing reads (4 consecutive rows x 64 B per 32 lanes).
template <int D>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return c ^ (((r & 3) << 1) | ((r >> 2) & 1));
  }
}
// Element offset of (row r, column col) in a swizzled tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * D + 8 * swz_chunk<D>(r, col >> 3) + (col & 7);
}

// 16-byte read of 8 consecutive columns (col multiple of 8) of row r.
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* tile, int r, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_off<D>(r, col));
}

// Transposing read: an MFMA operand fragment holding, for lane l, the column
// `col0 + (l % 32)` of the 8 consecutive rows `row0 + 8*(l/32) .. +7`
// (the k-contiguous operand layout of v_mfma_*_32x32x16_bf16) out of a
// row-major tile.  Uses ds_read_b64_tr_b16: within each 16-lane group, lane s
// supplies the address of 4 columns of one row and lane i receives column i of
// 4 consecutive rows.
template <int D>
__device__ __forceinline__ bf16x8 lds_col8(const uint16_t* tile, int row0, int col0) {
  const int l = threadIdx.x & 63;
  const int grp = l >> 4, s = l & 15;
  const int r = row0 + 8 * (grp >> 1) + (s >> 2);
  const int c = col0 + 16 * (grp & 1) + 4 * (s & 3);
  const uint16_t* p0 = tile + tile_off<D>(r, c);
  const uint16_t* p1 = tile + tile_off<D>(r + 4, c);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row permutation used when a 32x32 MFMA output feeds the k-operand of the next
// MFMA: operand row m is loaded from tile row rho(m), so that output element r
// of lane l (MFMA row 8(r/4) + 4(l/32) + r%4) sits at tile row
// 16(r/8) + 8(l/32) + (r%8), i.e. the lane's 8 values for k-step ks are exactly
// the rows 16ks + 8(l/32) + e that the k-operand layout asks for.
__device__ __forceinline__ int rho(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}
// Tile row (within a 32-row subtile) of output element r for lane half h.
__device__ __forceinline__ int out_row(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

__device__ __forceinline__ float wave_max32(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float wave_sum32(float x) { return x + __shfl_xor(x, 32, 64); }

// ------------------------------------------------------ gathered key tiles
// Number of valid (>= 0) entries of a group list; -1 entries only trail.
template <int NT>
__device__ __forceinline__ int count_valid(const int32_t* g, int kg, int* sgid) {
  int nv = 0;
  for (int i0 = 0; i0 < kg; i0 += NT) {
    const int i = i0 + threadIdx.x;
    int v = -1;
    if (i < kg) { v = g[i]; sgid[i] = v; }
    nv += __syncthreads_count(v >= 0);
  }
  return nv;
}

// Global -> register -> LDS staging of one 64-token K (and V) tile.
template <int D, int NT>
struct TileLoader {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int NCH = 64 * CH;               // chunks per tensor tile
  static constexpr int LPT = (NCH + NT - 1) / NT;   // chunks per thread per tensor
  uint4 rk[LPT], rv[LPT];

  // Token of tile row r: selected tiles map 8 groups, the last tile is the own chunk.
  __device__ __forceinline__ int64_t token(int t, int n_sel_tiles, int n_valid, const int* sgid,
                                           int J, int r) const {
    if (t < n_sel_tiles) {
      const int slot = 8 * t + (r >> 3);
      return slot < n_valid ? (int64_t)kGroup * sgid[slot] + (r & 7) : -1;
    }
    return (int64_t)kChunk * J + r;
  }
  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, int t, int n_sel_tiles,
                                       int n_valid, const int* sgid, int J) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int idx = threadIdx.x + i * NT;
      const int r = idx / CH, c = idx % CH;
      const int64_t tok = idx < NCH ? token(t, n_sel_tiles, n_valid, sgid, J, r) : -1;
      if (tok >= 0) {
        rk[i] = *reinterpret_cast<const uint4*>(kb + tok * D + 8 * c);
        rv[i] = *reinterpret_cast<const uint4*>(vb + tok * D + 8 * c);
      } else {
        rk[i] = make_uint4(0, 0, 0, 0);
        rv[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* tk, uint16_t* tv) const {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int idx = threadIdx.x + i * NT;
      if (NCH % NT != 0 && idx >= NCH) continue;
      const int r = idx / CH, c = idx % CH;
      const int off = r * D + 8 * swz_chunk<D>(r, c);
      *reinterpret_cast<uint4*>(tk + off) = rk[i];
      *reinterpret_cast<uint4*>(tv + off) = rv[i];
    }
  }
};

}  // namespace hga
