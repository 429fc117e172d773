// Device-side helpers shared by the HGA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void_t;

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

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Hardware round-to-nearest-even conversions (v_cvt_pk_bf16_f32), for the hot loops.
__device__ __forceinline__ bf16x8 f32x8_to_bf16x8(const float* x) {
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ uint2 f32x4_to_bf16x4_bits(float a, float b, float c, float d) {
  const f32x4v v = {a, b, c, d};
  return __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
}
// 2^x on the transcendental unit (inputs are softmax exponents <= 0; -inf gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Wait until every vector memory access issued by this wave has completed: loads,
// stores and global->LDS copies (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ------------------------------------------------ exchange between work-groups
// Values that a work-group of the same launch reads (possibly on another XCD, whose
// L2 is not coherent with this one) are written and read with these.
// Device-scope coherent stores and loads (relaxed atomics at agent scope).
__device__ __forceinline__ void put(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t get(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival of a work-group at a counter, after its put()s; true in the last of the n
// that arrive.  Every wave waits for its stores to complete first, so a work-group
// that sees the final count also sees every put() of the others.  The last one
// resets the counter for the next launch.  All threads of the work-group call it.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int n, int* flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_dma();   // s_waitcnt vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == (uint32_t)(n - 1);
    if (*flag) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag != 0;
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
// Transposing reads (ds_read_b64_tr_b16) produce the k-contiguous operand layout of
// v_mfma_*_32x32x16_bf16 out of a row-major tile: within each 16-lane group, lane s
// supplies the address of 4 columns of one row and lane i receives column i of 4
// consecutive rows; two such reads give a lane the column `col0 + (l % 32)` of the 8
// rows `row0 + 8*(l/32) .. +7`.

// Swizzle term of tile row r (depends on r % 16 only).
template <int D>
__device__ __forceinline__ int swz_f(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 1) | ((r >> 2) & 1);
}

// A per-lane value the compiler must treat as freshly computed: addresses derived
// from it are rebuilt where they are used instead of being hoisted out of the
// tile loop, each one pinning a register for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Row-fragment reader for one lane: rows `row` (fixed per lane) of a swizzled
// tile, 8 columns at a time.
template <int D>
struct RowReader {
  int base, f;   // element offset of the row, swizzle term
  __device__ __forceinline__ RowReader(int row) {
    const int r = opaque(row);
    base = r * D;
    f = swz_f<D>(r);
  }
  __device__ __forceinline__ bf16x8 operator()(const uint16_t* tile, int col) const {
    return *reinterpret_cast<const bf16x8*>(tile + base + 8 * ((col >> 3) ^ f));
  }
};

// Transposing fragment reader (see above) for row blocks starting at a multiple
// of 16: lane-constant parts precomputed once per use site.
template <int D>
struct ColReader {
  int rr, cc, f0, f1;
  __device__ __forceinline__ ColReader() {
    const int l = opaque(threadIdx.x & 63);
    const int grp = l >> 4, s = l & 15;
    rr = 8 * (grp >> 1) + (s >> 2);
    cc = 16 * (grp & 1) + 4 * (s & 3);
    f0 = swz_f<D>(rr);
    f1 = swz_f<D>(rr + 4);
  }
  // column col0 + (l % 32) of rows row0 + 8 (l / 32) .. +7; row0 % 16 == 0, col0 % 32 == 0
  __device__ __forceinline__ bf16x8 operator()(const uint16_t* tile, int row0, int col0) const {
    const int c = (col0 + cc) >> 3, sub = cc & 7;
    const uint16_t* p0 = tile + (row0 + rr) * D + 8 * (c ^ f0) + sub;
    const uint16_t* p1 = tile + (row0 + rr + 4) * D + 8 * (c ^ f1) + sub;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Per-lane LDS byte offsets of a wave's fragment reads, computed once per kernel.
// refresh() passes them through an empty asm in place before each tile: the compiler
// then neither hoists one address per (buffer, fragment) out of the tile loop nor
// recomputes them, and the constant part of every address (buffer, k-step) folds
// into the instruction's immediate offset.
template <int N>
struct LaneOffsets {
  int o[N];
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(o[i]));
  }
};

// Row reads (operand A/B layout): row `row` of a swizzled tile, 8 columns at
// 16 ks + 8 h for k-step ks; `extra` (bytes, compile-time) moves to another row block.
template <int D>
struct RowOffsets : LaneOffsets<D / 16> {
  __device__ __forceinline__ void init(int row, int h) {
    const int f = swz_f<D>(row);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) this->o[ks] = 2 * (row * D + 8 * ((2 * ks + h) ^ f));
  }
  template <int EXTRA = 0>
  __device__ __forceinline__ bf16x8 read(const uint16_t* tile, int ks) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + EXTRA + this->o[ks]);
  }
};

// Transposing reads (see above): the fragment of rows 16 ks .. +15 and columns
// 32 dt .. +31; the row block moves by an immediate, the column tile picks an offset.
template <int D>
struct ColOffsets : LaneOffsets<D / 16> {   // [2 dt + 0/1]: the two 4-row halves
  __device__ __forceinline__ void init(int l) {
    const int grp = l >> 4, s = l & 15;
    const int rr = 8 * (grp >> 1) + (s >> 2), cc = 16 * (grp & 1) + 4 * (s & 3);
    const int f0 = swz_f<D>(rr), f1 = swz_f<D>(rr + 4);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int c = (32 * dt + cc) >> 3;
      this->o[2 * dt] = 2 * (rr * D + 8 * (c ^ f0) + (cc & 7));
      this->o[2 * dt + 1] = 2 * ((rr + 4) * D + 8 * (c ^ f1) + (cc & 7));
    }
  }
  template <int KS>
  __device__ __forceinline__ bf16x8 read(const uint16_t* tile, int dt) const {
    const char* t = reinterpret_cast<const char*>(tile) + 2 * 16 * KS * D;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + this->o[2 * dt]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + this->o[2 * dt + 1]));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Copies of gathered 64-row tiles into the swizzled layout, wave by wave.  Copy
// block bi (1 KiB, rows RPB*bi ..) lies inside group slot (RPB*bi)/8, so its source
// is one contiguous run: the slot's group (wave-uniform) plus a per-lane offset.
// NW waves share a tile's D/8 blocks; wave w copies blocks w, w + NW, ...
// The group offsets of the next tile to copy are fetched (scalar loads) one tile
// ahead, so their latency stays off the critical path.
template <int D, int NW>
struct GroupCopier {
  static constexpr int CH = D / 8, RPB = 64 / CH, NBLK = D / 8, BPW = NBLK / NW;
  static_assert(NBLK % NW == 0, "copy blocks split evenly over the waves");
  int64_t next[BPW];   // byte offset of the source group of each of this wave's blocks

  __device__ __forceinline__ static int slot(int k) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    return (RPB * (w + NW * k)) >> 3;
  }
  // group_of(slot) -> group id (wave-uniform) of the tile being prepared.
  template <typename GroupOf>
  __device__ __forceinline__ void fetch(const GroupOf& group_of) {
#pragma unroll
    for (int k = 0; k < BPW; ++k) next[k] = (int64_t)group_of(slot(k)) * (8 * D * 2);
  }
  // Copy of this wave's block number k (0 .. BPW-1) of the prepared tile.
  template <int K>
  __device__ __forceinline__ void copy_one(uint16_t* tile, const char* base) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int bi = w + NW * K;
    const int r = RPB * bi + l / CH;
    const uint32_t lane_off = 2u * (uint32_t)((((RPB * bi) & 7) + l / CH) * D + 8 * swz_chunk<D>(r, l % CH));
    __builtin_amdgcn_global_load_lds((const void*)(base + next[K] + lane_off), (lds_void_t*)(tile + 512 * bi), 16, 0, 0);
  }
};

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

// The same reductions over lanes l and l ^ 32 with v_permlane32_swap (a VALU op, no
// LDS round trip): swapping a value with itself leaves the lower half's values in
// the first result and the upper half's in the second, in every lane.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + x.lo + x.hi for a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_bf16x2(uint32_t x, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}

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

// Copies per wave of one dma_tile call when NW waves share it (waves beyond the
// tile's D/8 blocks issue none).
template <int D, int NW>
constexpr int dma_per_wave() { return (D / 8) >= NW ? (D / 8) / NW : 1; }

// Asynchronous global -> LDS copy of one 64-row tile into the swizzled layout
// (global_load_lds_dwordx4: lane L of a wave writes the 16 bytes it loaded to
// LDS base + 16 L).  The tile is 64*D*2 bytes = D/8 blocks of 1 KiB; the NW waves
// split the blocks, and each lane fetches the logical chunk that belongs at its
// physical slot (the swizzle is an involution).  row_src(r) is the global address
// of tile row r.  Completion: s_waitcnt vmcnt(0) of the issuing wave, then a barrier.

template <int D, int NW, typename RowSrc>
__device__ __forceinline__ void dma_tile(uint16_t* tile, const RowSrc& row_src) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int RPB = 64 / CH;       // rows per 1 KiB block
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int bi = w; bi < CH; bi += NW) {
    const int r = RPB * bi + l / CH;
    const int c = swz_chunk<D>(r, l % CH);
    __builtin_amdgcn_global_load_lds((const void*)(row_src(r) + 8 * c), (lds_void_t*)(tile + 512 * bi), 16, 0, 0);
  }
}

// ------------------------------------------------------ a wave's 32 query rows
// A wave's 32 query rows (lane n = l & 31 holds row n in the MFMA output layout, the
// lane halves h the column halves) are contiguous in the row-major [.., rows, D]
// tensors.  Stored straight from that layout, every store instruction touches 32
// rows; through a private 32-row LDS region (16-byte chunks XOR-swizzled by row)
// every instruction writes whole rows instead.

// Store of a wave's 32 output rows dst .. dst + 31 (D bf16 each) through a 32-row
// region: val(dt, g) gives the lane's four bf16 values of its row at columns
// 32 dt + 8 g + 4 h .. +3 (the MFMA output layout) as a uint2.  The region must not
// be in use by another wave.
template <int D, typename Val>
__device__ __forceinline__ void store_rows32(uint16_t* region, uint16_t* dst, Val&& val) {
  constexpr int CH = D / 8, RPI = 64 / CH;   // chunks per row, rows per store
  const int l = threadIdx.x & 63, n = l & 31, h = l >> 5;
  const int f = swz_f<D>(n);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint2*>(region + n * D + 8 * ((4 * dt + g) ^ f) + 4 * h) = val(dt, g);
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = RPI * it + l / CH, c = l % CH;
    const uint4 x = *reinterpret_cast<const uint4*>(region + r * D + 8 * (c ^ swz_f<D>(r)));
    *reinterpret_cast<uint4*>(dst + (int64_t)r * D + 8 * c) = x;
  }
}


// s_waitcnt lgkmcnt(0) alone: this wave's LDS accesses have completed.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(N) for a compile-time N (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int I>
using ic = std::integral_constant<int, I>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// Work-group barrier for the tile pipelines.  __syncthreads() carries a release
// fence that makes the compiler wait for every outstanding vector-memory operation
// (s_waitcnt vmcnt(0)), which would drain the copies of the tiles still in flight.
// Here each wave has already waited for its own copies of the tile about to be read
// (vmcnt(N) with the later tiles still pending), and its reads of the buffer about to
// be overwritten have been consumed; LDS is coherent within the work-group, so a bare
// s_barrier suffices.  The signal fences only stop the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void tile_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Software pipeline over n tiles with NBUF buffer sets and NBUF-1 tiles in flight.
// issue(t, ic<B>) starts the asynchronous copies of tile t into buffer set B;
// with PREISSUED the caller has already issued tiles 0 .. NBUF-2 (those below n)
// into sets 0 .. NBUF-2, each wave with the same L copies per tile;
// compute(t, ic<B>) consumes buffer set B.  Every wave issues exactly L copies
// per tile (or none at all), so "tile t has landed" is vmcnt(L * tiles issued
// after t).  Buffer sets must be distinct LDS arrays chosen at compile time: the
// compiler then knows that reading one set never aliases copies into another
// and adds no wait of its own.  One barrier per tile: before tile t+NBUF-1 is
// issued into the set of tile t-1, every wave has finished computing tile t-1.
template <int NBUF, int L, bool PREISSUED = false, typename Issue, typename Compute>
__device__ __forceinline__ void pipeline(int n, Issue&& issue, Compute&& compute) {
  static_assert(NBUF >= 2 && NBUF <= 4, "2 to 4 buffer sets");
  constexpr int P = NBUF - 1;
  if constexpr (!PREISSUED) {
    static_for<0, P>([&](auto B) {
      if (B() < n) issue(B(), B);
    });
  }
  for (int t0 = 0; t0 < n; t0 += NBUF) {
    static_for<0, NBUF>([&](auto B) {
      const int t = t0 + B();
      if (t < n) {
        const int ahead = min(P - 1, n - 1 - t);       // tiles already issued after t
        if constexpr (P >= 3) {
          if (ahead >= 2) wait_vmcnt<2 * L>();
          else if (ahead == 1) wait_vmcnt<L>();
          else wait_vmcnt<0>();
        } else if constexpr (P == 2) {
          if (ahead >= 1) wait_vmcnt<L>();
          else wait_vmcnt<0>();
        } else {
          wait_vmcnt<0>();
        }
        tile_barrier();
        if (t + P < n) issue(t + P, ic<(B() + P) % NBUF>{});
        compute(t, B);
      }
    });
  }
}

}  // namespace hga
