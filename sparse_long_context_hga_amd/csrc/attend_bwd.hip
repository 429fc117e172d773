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
// bf16 path: three kernels, deterministic (no floating-point atomics):
//  * dq (query-major, one work-group per (sequence, KV head, query block) and
//    query-head slice): the forward's gathered tiles again; recomputes P from
//    LSE; writes dQ, and D = rowsum(dO * O) and -LSE log2(e) (workspace) for the
//    dK/dV kernel.  It
//    also inverts the selection for the active chunk of its own block -- the
//    ascending list of query blocks that attend the chunk -- and cuts the
//    chunk's work into 1..8 items of about 12 or 16 "rounds" (one round = the 64 rows
//    of one query head of one attending block), filed by size class;
//  * dkdv (one work-group per item, the largest size class first, so that the
//    grid starts with the heaviest items): the chunk's 64 keys and values stay in
//    registers; the item's rounds stream Q / dO rows through swizzled LDS; dK,
//    dV accumulate in fp32 registers (dV^T += dO^T P, dK^T += Q^T dS, the
//    transposing LDS reads supplying the k-contiguous operands); a chunk done
//    by one item writes bf16 dK/dV, otherwise each item writes an fp32 partial;
//  * finalize: sums a chunk's partials in item order and writes bf16 dK/dV, and
//    returns the class counts to zero for the next call.
// fp32 path: two plain SIMT kernels (dQ, dK/dV), fp32 throughout.
#include <hip/hip_ext.h>

#include "hga_device.h"
#include "hga_internal.h"

#include <math.h>

namespace hga {
namespace {

constexpr int kStages = 2;   // K/V tile buffer sets of the dQ kernel

constexpr int kMaxBlocks = 1024;   // query blocks per segment supported by the dkdv kernel
// dK/dV work is cut into items of about this many rounds.  Longer items mean fewer
// items (each pays a start-up and an epilogue of a few microseconds) but a longer
// slowest item.  The segment's own blocks attend its chunks more often when the
// history is short, so the chunks carry more rounds and longer items pay: measured
// on the 32-query / 8-KV-head layer, 12 is fastest with 14,336 history tokens per
// 2,048-token segment and 16 with 2,048 (8 to 32 tried).
constexpr int kTargetRoundsLongHistory = 12;
constexpr int kTargetRoundsShortHistory = 16;
constexpr int kMaxParts = 8;       // at most this many items per active chunk
constexpr int kClasses = 16;       // work-list size classes (rounds per work item, capped at 15)

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
  float* dvec;      // [B, Hq, S] rowsum(dO * O)            (workspace)
  float* nlse;      // [B, Hq, S] -LSE * log2(e), the exponent offset of P in base 2 (workspace)
  int* flags;       // [B, Hkv, S/64] number of work items of the chunk's dK/dV (workspace)
  int* vis;         // [B, Hkv, S/64, S/64] attending blocks, ascending: block | group mask << 16
  int* cls_count;   // [kClasses] work items filed per size class; zero between calls (workspace start)
  int4* cls_items;  // [kClasses, B*Hkv*S/64*kMaxParts] the items of each class, each {unit * kMaxParts +
                    // part, parts of the unit, visits of the unit, the block of the item's first round}
  float* parts;     // [B, Hkv, S/64, kMaxParts, 2, 64, d] fp32 partials (workspace)
  int64_t t_cap, t_hist, seg_len;
  int Hq, Hkv, kg, nb, n_units;
  int target_rounds;   // dK/dV rounds per work item (see kTargetRounds*)
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

// Inverse of the selection for the active segment, for active chunk cc of
// (sequence, KV head) bh: the ascending list of query blocks that attend it (its own
// block, causally, and every later block whose group list holds one of its 8
// groups), with the mask of the selected groups, and into how many work items its
// dK/dV is cut.  Runs inside the dQ kernel (one of the work-groups of unit (bh, cc))
// before its tile pipeline; gv holds this thread's first group ids of the later
// blocks, loaded early so that their latency overlaps the dQ kernel's own loads.
// The chunk's work items go to LDS (item_cls[k]: size class of item k, or -1 past
// the last item; item_entry[k]: its work-list entry) for the caller to file.
constexpr int kPlanLoads = 8;
template <int NT, int G>
__device__ __forceinline__ void plan_chunk(const BwdArgs& a, int bh, int cc, const int32_t (&gv)[kPlanLoads],
                                           uint32_t* mask, int* item_cls, int4* item_entry) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int64_t g_lo = (a.t_hist / kChunk + cc) * 8;
  const int32_t* g0 = a.gidx + ((int64_t)bh * a.nb + cc + 1) * a.kg;
  const int total = (a.nb - 1 - cc) * a.kg;
  auto mark = [&](int e, int64_t gid) __attribute__((always_inline)) {
    if (gid >= g_lo && gid < g_lo + 8) atomicOr(&mask[cc + 1 + e / a.kg], 1u << (int)(gid - g_lo));
  };
#pragma unroll
  for (int u = 0; u < kPlanLoads; ++u) mark(NT * u + tid, gv[u]);
  for (int e0 = NT * kPlanLoads; e0 < total; e0 += NT * kPlanLoads) {   // long segments only
    int32_t gx[kPlanLoads];
#pragma unroll
    for (int u = 0; u < kPlanLoads; ++u) {
      const int e = e0 + NT * u + tid;
      gx[u] = e < total ? g0[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPlanLoads; ++u) mark(e0 + NT * u + tid, gx[u]);
  }
  __syncthreads();
  if (w != 0) return;
  const int unit = bh * a.nb + cc;
  int n = 0;
  int* out = a.vis + (int64_t)unit * a.nb;
  for (int j0 = cc; j0 < a.nb; j0 += 64) {
    const int jj = j0 + l;
    const uint32_t m = jj < a.nb ? mask[jj] : 0u;
    const uint64_t bal = __ballot(m != 0u);
    const int at = n + __popcll(bal & ((1ull << l) - 1ull));
    if (m != 0u) {
      out[at] = jj | (int)(m << 16);
      // The list again in LDS, from mask[cc] on: at <= jj - cc, so this overwrites only
      // entries this wave has already read.
      mask[cc + at] = (uint32_t)jj;
    }
    n += __popcll(bal);
  }
  // G rounds (query heads) per attending block (n >= 1: the own block), cut into np
  // items of about a.target_rounds; item k starts at round k * rounds / np, and its
  // size class is its number of rounds (capped).  The entry carries the block of the
  // item's first round, so that the dK/dV kernel can start its copies before it has
  // read the visit list.
  const int rounds = G * n;
  const int np = min(kMaxParts, (rounds + a.target_rounds - 1) / a.target_rounds);
  if (l < kMaxParts) {
    item_cls[l] = l < np ? min(kClasses - 1, (l + 1) * rounds / np - l * rounds / np) : -1;
    if (l < np) item_entry[l] = make_int4(unit * kMaxParts + l, np, n, (int)mask[cc + (l * rounds / np) / G]);
  }
  if (l == 0) a.flags[unit] = np;
}

// ---------------------------------------------------------------- dQ (bf16)
// HPW query heads of the G sharing a KV head per work-group (as in the forward).
template <int D, int G, int HPW>
__global__ __launch_bounds__(128 * HPW, 8 / (2 * HPW) > 1 ? 8 / (2 * HPW) : 1)
void attend_bwd_dq_bf16_kernel(BwdArgs a) {
  constexpr int NT = 128 * HPW;
  constexpr int NW = 2 * HPW;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
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
  const int J = (int)(a.t_hist / kChunk) + j;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n = l & 31;
  const int hh = (item % (G / HPW)) * HPW + (w >> 1);
  const int pos = 32 * (w & 1) + n;
  // First row of this wave's 32 (wave-uniform) and this lane's row.
  const int64_t qrow0 = (((int64_t)b * a.Hq + kvh * G + hh) * a.seg_len) + (int64_t)j * kQBlock + 32 * (w & 1);
  const int64_t qrow = qrow0 + n;
  const uint16_t* kb = (const uint16_t*)a.k + (int64_t)bh * a.t_cap * D;
  const uint16_t* vb = (const uint16_t*)a.v + (int64_t)bh * a.t_cap * D;
  // 32-row LDS region of wave wv in the two tile buffer sets (for dQ after the last
  // tile).
  auto row_region = [&](int wv) __attribute__((always_inline)) -> uint16_t* {
    uint16_t* base = (wv >> 1) == 0 ? k0 : (wv >> 1) == 1 ? v0 : (wv >> 1) == 2 ? k1 : v1;
    return base + (wv & 1) * 32 * D;
  };

  // The selection inverse of active chunk j: its group ids are loaded first (their
  // latency overlaps the loads below), used after the group list is in LDS.
  __shared__ uint32_t pmask[kMaxBlocks];
  const bool do_plan = item % (G / HPW) == 0;
  int32_t pgv[kPlanLoads];
  {
    const int32_t* g0 = a.gidx + ((int64_t)bh * a.nb + j + 1) * a.kg;
    const int total = (a.nb - 1 - j) * a.kg;
#pragma unroll
    for (int u = 0; u < kPlanLoads; ++u) {
      const int e = NT * u + tid;
      pgv[u] = do_plan && e < total ? g0[e] : -1;
    }
    if (do_plan)
      for (int i = tid; i < a.nb; i += NT) pmask[i] = i == j ? 0xFFu : 0u;   // ordered by the barrier below
  }

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
  const float Dr = half_sum(dpart);
  const float lse2 = a.lse[qrow] * kLog2e;
  if (h == 0) {
    a.dvec[qrow] = Dr;
    a.nlse[qrow] = -lse2;
  }

  const int n_valid = __builtin_amdgcn_readfirstlane(
      count_valid<NT>(a.gidx + (int64_t)unit * a.kg, a.kg, sgid));   // ends with a barrier
  __shared__ int item_cls[kMaxParts];
  __shared__ int4 item_entry[kMaxParts];
  if (do_plan) plan_chunk<NT, G>(a, bh, j, pgv, pmask, item_cls, item_entry);
  const int n_sel_tiles = (n_valid + 7) >> 3;
  const int n_tiles = n_sel_tiles + 1;
  // Tile t: 8 selected groups, or the own chunk as the last tile; slots past the
  // selection repeat the own chunk's first group (masked).
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
  constexpr int BPW = GroupCopier<D, NW>::BPW;
  auto issue = [&](int t, auto B) __attribute__((always_inline)) {
    static_for<0, BPW>([&](auto K) { copier.template copy_one<K()>(KB(B), (const char*)kb); });
    static_for<0, BPW>([&](auto K) { copier.template copy_one<K()>(VB(B), (const char*)vb); });
    if (t + 1 < n_tiles) prepare(t + 1);
  };
  prepare(0);
  RowOffsets<D> kro;      // K / V rows rho(n) (+32 rows for the second subtile as an immediate)
  kro.init(rho(n), h);
  ColOffsets<D> kco;      // K^T fragments
  kco.init(l);

  const float c2 = a.scale * kLog2e;
  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = f32x16{};

  auto compute = [&](int t, auto B) __attribute__((always_inline)) {
    const uint16_t* K = KB(B);
    const uint16_t* V = VB(B);
    kro.refresh();
    kco.refresh();
    const bool local = t == n_sel_tiles;
    const bool full = !local && 8 * (t + 1) <= n_valid;
    const int kv_lim = full ? 63 : local ? pos : 8 * (n_valid - 8 * t) - 1;
    // One 32-key subtile at a time keeps the live score registers to 2 x 16.
    static_for<0, 2>([&](auto KT) {
      constexpr int kt = KT();
      f32x16 s = {}, dpv = {};
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {               // two batches of KS/2 k-steps
        bf16x8 ka[KS / 2], va[KS / 2];
#pragma unroll
        for (int i = 0; i < KS / 2; ++i) {
          ka[i] = kro.template read<kt * 32 * D * 2>(K, hb * KS / 2 + i);
          va[i] = kro.template read<kt * 32 * D * 2>(V, hb * KS / 2 + i);
        }
#pragma unroll
        for (int i = 0; i < KS / 2; ++i) {
          s = mfma32(ka[i], qf[hb * KS / 2 + i], s);
          dpv = mfma32(va[i], dof[hb * KS / 2 + i], dpv);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
      }
      // K^T fragments for the dQ update (independent of dS: read before the softmax math).
      bf16x8 kt_fr[2][DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        kt_fr[0][dt] = kco.template read<2 * kt>(K, dt);
        kt_fr[1][dt] = kco.template read<2 * kt + 1>(K, dt);
      }

      // Mask only the own chunk and a partial last tile (a score of -inf gives P = 0).
      // The empty asm keeps this a branch, so that full tiles skip the compares.
      if (!full) {
        asm volatile("" ::: "memory");
        const int thr = kv_lim - 32 * kt - 8 * h;   // out_row(r, h) + 32 kt > kv_lim  <=>  out_row(r, 0) > thr
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (out_row(r, 0) > thr) s[r] = -INFINITY;
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(fmaf(s[r], c2, -lse2)) * (dpv[r] - Dr);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 dsf = f32x8_to_bf16x8(ds + 8 * half);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dqacc[dt] = mfma32(kt_fr[half][dt], dsf, dqacc[dt]);
      }
    });
  };

  pipeline<kStages, 2 * BPW>(n_tiles, issue, compute);

  // File the chunk's work items under their size classes, at the positions an
  // atomic count of each class gives them (the order within a class is immaterial:
  // every item writes its own output or partial).  Only the dK/dV kernel reads
  // them, so this waits until the tiles are done, and the atomics' round trip
  // overlaps the dQ stores below.
  int pcls = -1;
  uint32_t pslot = 0;
  if (do_plan && threadIdx.x < kMaxParts) {
    pcls = item_cls[threadIdx.x];
    if (pcls >= 0)
      pslot = (uint32_t)__hip_atomic_fetch_add(a.cls_count + pcls, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // dQ leaves through this wave's 32-row LDS region as whole rows; the barrier keeps
  // every region free until all waves have finished their last tile.
  tile_barrier();
  store_rows32<D>(row_region(w), (uint16_t*)a.dq + qrow0 * D, [&](int dt, int g) __attribute__((always_inline)) {
    return f32x4_to_bf16x4_bits(dqacc[dt][4 * g] * a.scale, dqacc[dt][4 * g + 1] * a.scale,
                                dqacc[dt][4 * g + 2] * a.scale, dqacc[dt][4 * g + 3] * a.scale);
  });
  const uint32_t cap = (uint32_t)a.n_units * kMaxParts;
  if (pcls >= 0 && pslot < cap)   // (always below cap when the counts started the call at zero)
    a.cls_items[(int64_t)pcls * cap + pslot] = item_entry[threadIdx.x];
}

// ---------------------------------------------------------------- dK/dV (bf16)
// Work item (sequence, KV head, active chunk, part).  A chunk is attended by its
// own block (causally) and by every later block whose selection holds one of its
// groups; each such block contributes G "rounds" (64 rows of one query head).
// The dQ kernel cuts a chunk's rounds into np = min(kMaxParts, ceil(rounds /
// target_rounds)) contiguous slices.  With np = 1 the item writes bf16 dK/dV
// itself; otherwise every item writes an fp32 partial, summed in part order by
// the finalize kernel (deterministic; no atomics).
// Inside a work-group: 4 waves; wave w owns keys 32*(w&1) .. +31 of the chunk
// and rows 32*(w>>1) .. +31 of every round; each round's Q/dO rows are copied
// into LDS one round ahead of their use (two buffer sets: a deeper prefetch puts
// more copies in flight per CU, and those delay the ones the current round waits
// for).

// Workspace layout (byte offsets).  The class counts come first, at the same place
// for every shape, so that a workspace reused across shapes keeps them at zero.
struct DkdvLayout {
  static size_t up(size_t x) { return (x + 255) & ~(size_t)255; }
  static constexpr size_t dvec_off = 256;   // after the kClasses counts
  static size_t nlse_off(size_t rows) { return up(dvec_off + rows * 4); }
  static size_t flags_off(size_t rows) { return up(nlse_off(rows) + rows * 4); }
  static size_t vis_off(size_t rows, size_t units) { return up(flags_off(rows) + units * 4); }
  static size_t items_off(size_t rows, size_t units, size_t nb) { return up(vis_off(rows, units) + units * nb * 4); }
  static size_t part_off(size_t rows, size_t units, size_t nb) {
    return up(items_off(rows, units, nb) + kClasses * units * kMaxParts * sizeof(int4));
  }
};
static_assert(kClasses * sizeof(int) <= DkdvLayout::dvec_off, "class counts fit ahead of the row vectors");

template <int D, int G>
__global__ __launch_bounds__(256, 1) void attend_bwd_dkdv_bf16_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  __shared__ __align__(16) uint16_t q0[64 * D], do0[64 * D], q1[64 * D], do1[64 * D];
  __shared__ __align__(16) float ls0[64], dr0[64], ls1[64], dr1[64];
  __shared__ uint32_t vmask[kMaxBlocks];   // group mask of the i-th attending block
  __shared__ int vlist[kMaxBlocks];        // i-th attending block
  auto QB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return q0; else return q1;
  };
  auto OB = [&](auto B) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (B() == 0) return do0; else return do1;
  };
  auto LB = [&](auto B) __attribute__((always_inline)) -> float* {
    if constexpr (B() == 0) return ls0; else return ls1;
  };
  auto RB = [&](auto B) __attribute__((always_inline)) -> float* {
    if constexpr (B() == 0) return dr0; else return dr1;
  };

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = l & 31;
  // Work item number blockIdx.x in the order of size classes, largest first (items
  // that finish early leave their compute unit to the next ones, so the long items
  // go first): the classes' counts locate the item's class and its place in it.
  const uint32_t cap = (uint32_t)a.n_units * kMaxParts;
  int4 entry;
  {
    const int c = l < kClasses ? a.cls_count[kClasses - 1 - l] : 0;   // lane l: the l-th largest class
    int incl = c;
#pragma unroll
    for (int off = 1; off < kClasses; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (l >= off) incl += y;
    }
    const uint64_t past = __ballot(l < kClasses && incl > (int)blockIdx.x);
    if (past == 0) return;                          // beyond the last item
    const int f = __builtin_ctzll(past);
    const uint32_t at = (uint32_t)((int)blockIdx.x - __shfl(incl - c, f, 64));
    if (at >= cap) return;                          // (counts that did not start at zero)
    entry = a.cls_items[(int64_t)(kClasses - 1 - f) * cap + at];
  }
  const int item = __builtin_amdgcn_readfirstlane(entry.x);
  const int np = __builtin_amdgcn_readfirstlane(entry.y);
  const int n_visits = __builtin_amdgcn_readfirstlane(entry.z);
  const uint32_t first = (uint32_t)__builtin_amdgcn_readfirstlane(entry.w);
  if (item < 0) return;
  const int part = item % kMaxParts;
  const int unit = item / kMaxParts;
  if (unit >= a.n_units || part >= np || n_visits > a.nb) return;   // not an item of this selection
  if (first >= (uint32_t)a.nb) return;             // (unsigned: no negative block either)
  const int cc = unit % a.nb;                      // active chunk == its own query block
  const int bh = unit / a.nb;
  const int b = bh / a.Hkv, kvh = bh % a.Hkv;
  const int64_t cglob = a.t_hist / kChunk + cc;    // global chunk id
  // Wave w owns keys 32*(w&1) .. +31 and rows 32*(w>>1) .. +31 of every round; the
  // two row halves are summed at the end.
  const int kh = w & 1, rh = w >> 1;
  const int key = 32 * kh + n;                     // this lane's key (operand-B column)

  // This item's slice of the chunk's rounds (round r = attending block r / G, query head r % G).
  const int rounds = G * n_visits;
  const int r_lo = part * rounds / np, r_hi = (part + 1) * rounds / np;

  const uint16_t* qg = (const uint16_t*)a.q;
  const uint16_t* dg = (const uint16_t*)a.d_o;
  auto round_row0 = [&](int r, int jj) __attribute__((always_inline)) -> int64_t {
    return (((int64_t)b * a.Hq + kvh * G + r % G) * a.seg_len) + (int64_t)jj * kQBlock;
  };
  // Round: the 64 rows of one query head of one attending block -> Q, dO tiles,
  // -LSE log2(e), D.  Every wave copies the 64 values of each itself (identical data), so that all
  // waves issue the same number of copies per round.
  auto issue_rows = [&](int64_t row0, auto B) __attribute__((always_inline)) {
    dma_tile<D, 4>(QB(B), [&](int rr) { return qg + (row0 + rr) * D; });
    dma_tile<D, 4>(OB(B), [&](int rr) { return dg + (row0 + rr) * D; });
    __builtin_amdgcn_global_load_lds((const void*)(a.nlse + row0 + l), (lds_void_t*)LB(B), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(a.dvec + row0 + l), (lds_void_t*)RB(B), 4, 0, 0);
  };
  auto issue = [&](int i, auto B) __attribute__((always_inline)) {
    issue_rows(round_row0(r_lo + i, vlist[(r_lo + i) / G]), B);
  };
  // Everything the first round needs travels at once: the visit list (into
  // registers), the first round's rows (its block comes with the work-list entry) and
  // the chunk's K and V rows (coalesced copies into buffer set 1, which the second
  // round uses later).  The second round's rows follow once these have landed, from
  // the pipeline: every CU loads at the same moment, and copies still in flight would
  // share the bandwidth with the ones the first round waits for.
  int vv[kMaxBlocks / 256];
#pragma unroll
  for (int k = 0; k < kMaxBlocks / 256; ++k) {
    const int i = tid + 256 * k;
    vv[k] = i < n_visits ? a.vis[(int64_t)unit * a.nb + i] : 0;
  }
  issue_rows(round_row0(r_lo, (int)first), ic<0>{});
  {
    const uint16_t* kp = (const uint16_t*)a.k + ((int64_t)bh * a.t_cap + cglob * kChunk) * D;
    const uint16_t* vp = (const uint16_t*)a.v + ((int64_t)bh * a.t_cap + cglob * kChunk) * D;
    dma_tile<D, 4>(q1, [&](int rr) { return kp + (int64_t)rr * D; });
    dma_tile<D, 4>(do1, [&](int rr) { return vp + (int64_t)rr * D; });
  }
  constexpr int L = 2 * dma_per_wave<D, 4>() + 2;   // copies per wave per round
#pragma unroll
  for (int k = 0; k < kMaxBlocks / 256; ++k) {
    const int i = tid + 256 * k;
    if (i < n_visits) {
      // entries come from the dQ kernel's selection inverse; a block id outside the
      // segment (never written that way) is clamped and masked out rather than read
      const int jj = vv[k] & 0xFFFF;
      vlist[i] = min(jj, a.nb - 1);
      vmask[i] = jj < a.nb ? (uint32_t)vv[k] >> 16 : 0u;
    }
  }
  // This wave's share of the copies has landed; after the barrier every wave's share
  // and the visit list are in LDS.
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  tile_barrier();
  bf16x8 kf[KS], vf[KS];
  {
    RowOffsets<D> kvo;   // key row 32 kh + n
    kvo.init(key, h);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = kvo.read(q1, ks);
      vf[ks] = kvo.read(do1, ks);
    }
  }
  wait_lgkmcnt0();   // read before the pipeline's first barrier lets set 1 be refilled

  const float c2 = a.scale * kLog2e;
  f32x16 dvacc[DT], dkacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) { dvacc[dt] = f32x16{}; dkacc[dt] = f32x16{}; }
  // Per-lane LDS offsets of the fragment reads, computed once: row reads of this
  // wave's rows 32 rh + rho(n); transposing reads of its 32-row half (the swizzle
  // repeats every 16 rows, so the half is a plain shift of the offsets).
  RowOffsets<D> rowo;
  rowo.init(32 * rh + rho(n), h);
  ColOffsets<D> colo;
  colo.init(l);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) colo.o[i] += 2 * 32 * rh * D;

  auto compute = [&](int i, auto B) __attribute__((always_inline)) {
    const uint16_t* tq = QB(B);
    const uint16_t* tdo = OB(B);
    const float* nls = LB(B);
    const float* drv = RB(B);
    const int vi = (r_lo + i) / G;
    // the round's block and group mask are the same for every lane
    const bool own = __builtin_amdgcn_readfirstlane(vlist[vi]) == cc;
    const uint32_t vm = (uint32_t)__builtin_amdgcn_readfirstlane((int)vmask[vi]);
    // A later block that selected none of this wave's 4 groups adds nothing to its keys.
    if (!own && ((vm >> (4 * kh)) & 0xFu) == 0u) return;
    const bool key_on = ((vm >> (key >> 3)) & 1u) != 0u;
    rowo.refresh();
    colo.refresh();
    f32x16 s = {}, dpv = {};
    {
      // All row fragments first, then the MFMAs: the reads overlap each other and the
      // first MFMAs instead of each read waiting out the LDS latency alone.
      bf16x8 qa[KS], da[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[ks] = rowo.read(tq, ks);
        da[ks] = rowo.read(tdo, ks);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(qa[ks], kf[ks], s);
        dpv = mfma32(da[ks], vf[ks], dpv);
      }
      // One batch: every read, then every MFMA.  (While copies into LDS are in flight
      // the compiler can only wait for all outstanding LDS reads at once.)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
    }
    static_for<0, 2>([&](auto KSI) {                 // rows 16ks .. 16ks+15 of the wave's 32
      constexpr int ks = KSI();
      // Transposed fragments of dO and Q for these rows (independent of P: issued first).
      bf16x8 fo[DT], fq[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        fo[dt] = colo.template read<ks>(tdo, dt);
        fq[dt] = colo.template read<ks>(tq, dt);
      }
      // -LSE log2(e) and D of the 8 consecutive rows this lane holds (two 16-byte LDS reads each).
      const int row0 = 32 * rh + 16 * ks + 8 * h;
      const f32x4v l0 = *reinterpret_cast<const f32x4v*>(nls + row0);
      const f32x4v l1 = *reinterpret_cast<const f32x4v*>(nls + row0 + 4);
      const f32x4v d0 = *reinterpret_cast<const f32x4v*>(drv + row0);
      const f32x4v d1 = *reinterpret_cast<const f32x4v*>(drv + row0 + 4);
      // Row row0 + e sees this lane's key iff e >= thr: in the own block causally
      // (key <= row), in a later block when the key's group is selected.
      const int thr = own ? key - row0 : key_on ? 0 : 8;
      float p[8], ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float nl = e < 4 ? l0[e & 3] : l1[e & 3];
        const float dr = e < 4 ? d0[e & 3] : d1[e & 3];
        const float pe = fast_exp2(fmaf(s[8 * ks + e], c2, nl));
        p[e] = e >= thr ? pe : 0.f;
        ds[e] = p[e] * (dpv[8 * ks + e] - dr);
      }
      const bf16x8 pf = f32x8_to_bf16x8(p);
      const bf16x8 dsf = f32x8_to_bf16x8(ds);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dvacc[dt] = mfma32(fo[dt], pf, dvacc[dt]);
        dkacc[dt] = mfma32(fq[dt], dsf, dkacc[dt]);
      }
    });
  };

  pipeline<2, L, /*PREISSUED=*/true>(r_hi - r_lo, issue, compute);

  // Sum the two row halves (waves 2,3 -> waves 0,1) through LDS; waves 0,1 then put
  // the sums, row-major by key, in their own halves' buffers, and all four waves
  // store them with whole-row (coalesced) writes: bf16 dK/dV when one item does the
  // chunk, this item's fp32 partial otherwise.  The halves sit in the stage buffers
  // (dV in q0/q1, dK in do0/do1, by key half); no copies are in flight after the last
  // round and every wave's reads of them have been consumed, so LDS-only barriers
  // suffice, and the global stores are never waited for.
  float* red_v = reinterpret_cast<float*>(kh == 0 ? q0 : q1);    // per key half: DT*16*64 floats
  float* red_k = reinterpret_cast<float*>(kh == 0 ? do0 : do1);
  static_assert(sizeof(q0) >= DT * 16 * 64 * sizeof(float), "reduction buffer");
  constexpr int C32 = D / 4, C16 = D / 8;   // 16-byte chunks per fp32 / bf16 row
  const bool split = np > 1;
  tile_barrier();
  // The halves travel as 16-byte pieces, lane-major: piece (dt, q) of lane l holds
  // accumulator elements 4q .. 4q+3 of tile dt.
  auto piece = [&](float* red, int dt, int q) __attribute__((always_inline)) -> float4* {
    return reinterpret_cast<float4*>(red) + (dt * 4 + q) * 64 + l;
  };
  if (rh == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *piece(red_v, dt, q) = make_float4(dvacc[dt][4 * q], dvacc[dt][4 * q + 1], dvacc[dt][4 * q + 2], dvacc[dt][4 * q + 3]);
        *piece(red_k, dt, q) = make_float4(dkacc[dt][4 * q], dkacc[dt][4 * q + 1], dkacc[dt][4 * q + 2], dkacc[dt][4 * q + 3]);
      }
  }
  wait_lgkmcnt0();
  tile_barrier();
  if (rh == 0) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 xv = *piece(red_v, dt, q), xk = *piece(red_k, dt, q);
        dvacc[dt][4 * q] += xv.x; dvacc[dt][4 * q + 1] += xv.y; dvacc[dt][4 * q + 2] += xv.z; dvacc[dt][4 * q + 3] += xv.w;
        dkacc[dt][4 * q] += xk.x; dkacc[dt][4 * q + 1] += xk.y; dkacc[dt][4 * q + 2] += xk.z; dkacc[dt][4 * q + 3] += xk.w;
      }
    // Row n (key 32 kh + n) of this half; the lane holds columns 32 dt + 8 g + 4 h .. +3.
    // Chunks are XOR-swizzled by row so that the 32 rows' writes spread over the banks.
    if (split) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = (8 * dt + 2 * g + h) ^ (n & (C32 - 1));
          *reinterpret_cast<float4*>(red_v + n * D + 4 * c) =
              make_float4(dvacc[dt][4 * g], dvacc[dt][4 * g + 1], dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]);
          *reinterpret_cast<float4*>(red_k + n * D + 4 * c) =
              make_float4(dkacc[dt][4 * g], dkacc[dt][4 * g + 1], dkacc[dt][4 * g + 2], dkacc[dt][4 * g + 3]);
        }
    } else {
      uint16_t* ov = reinterpret_cast<uint16_t*>(red_v);
      uint16_t* ok = reinterpret_cast<uint16_t*>(red_k);
      const float sc = a.scale;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int at = n * D + 8 * ((4 * dt + g) ^ (n & (C16 - 1))) + 4 * h;
          *reinterpret_cast<uint2*>(ov + at) =
              f32x4_to_bf16x4_bits(dvacc[dt][4 * g], dvacc[dt][4 * g + 1], dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]);
          *reinterpret_cast<uint2*>(ok + at) = f32x4_to_bf16x4_bits(
              dkacc[dt][4 * g] * sc, dkacc[dt][4 * g + 1] * sc, dkacc[dt][4 * g + 2] * sc, dkacc[dt][4 * g + 3] * sc);
        }
    }
  }
  wait_lgkmcnt0();
  tile_barrier();
  // Wave w stores the tile of (which = w >> 1: 0 dV, 1 dK; key half w & 1).
  const int which = w >> 1, half = w & 1;
  const char* src = reinterpret_cast<const char*>(which ? (half ? do1 : do0) : (half ? q1 : q0));
  if (split) {
    float* dst = a.parts + ((size_t)unit * kMaxParts + part) * (size_t)(2 * 64 * D) + (size_t)which * 64 * D +
                 (size_t)(32 * half) * D;
    constexpr int RPI = 64 / C32;   // rows per instruction
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int row = RPI * it + l / C32, c = l % C32;
      const float4 x = *reinterpret_cast<const float4*>(src + 16 * (row * C32 + (c ^ (row & (C32 - 1)))));
      *reinterpret_cast<float4*>(dst + (size_t)row * D + 4 * c) = x;
    }
  } else {
    uint16_t* dst = (uint16_t*)(which ? a.dk : a.dv) + ((int64_t)bh * a.seg_len + (int64_t)cc * kChunk + 32 * half) * D;
    constexpr int RPI = 64 / C16;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int row = RPI * it + l / C16, c = l % C16;
      const uint4 x = *reinterpret_cast<const uint4*>(src + 16 * (row * C16 + (c ^ (row & (C16 - 1)))));
      *reinterpret_cast<uint4*>(dst + (int64_t)row * D + 8 * c) = x;
    }
  }
}

// Sum the partials of chunks cut into several items, in item order, and write bf16
// dK/dV.  Work-group (chunk, slice): rows 8*slice .. +7 of dV and dK (512 float4s,
// two per thread); the loads of all partials are issued together.
constexpr int kFinalizeSlices = 8;

template <int D>
__global__ __launch_bounds__(256) void attend_bwd_dkdv_finalize_kernel(BwdArgs a) {
  // The dK/dV kernel has read the class counts: return them to zero for the next call.
  if (blockIdx.x == 0 && threadIdx.x < kClasses) a.cls_count[threadIdx.x] = 0;
  const int unit = blockIdx.x / kFinalizeSlices;
  const int slice = blockIdx.x % kFinalizeSlices;
  if (unit >= a.n_units) return;
  const int np = a.flags[unit];
  if (np <= 1) return;
  const float* part0 = a.parts + (size_t)unit * kMaxParts * (2 * 64 * D);
  const int cc = unit % a.nb;
  const int bh = unit / a.nb;
  const int64_t orow0 = (int64_t)bh * a.seg_len + (int64_t)cc * kChunk;
  constexpr int ROWS = 64 / kFinalizeSlices;
  constexpr int PER = 2 * ROWS * D / 4 / 256;      // float4s per thread
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f4 = threadIdx.x + 256 * i;           // float4 index within the slice
    const int which = f4 / (ROWS * D / 4);          // 0: dV, 1: dK
    const int within = (f4 % (ROWS * D / 4)) * 4 + slice * ROWS * D;   // element in the 64 x D tensor
    float4 x[kMaxParts];
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p)
      if (p < np) x[p] = *reinterpret_cast<const float4*>(part0 + (size_t)p * (2 * 64 * D) + (size_t)which * 64 * D + within);
    float4 acc = x[0];
#pragma unroll
    for (int p = 1; p < kMaxParts; ++p)
      if (p < np) { acc.x += x[p].x; acc.y += x[p].y; acc.z += x[p].z; acc.w += x[p].w; }
    const float sc = which ? a.scale : 1.f;
    uint16_t* out = (uint16_t*)(which ? a.dk : a.dv) + (orow0 + within / D) * D + within % D;
    *reinterpret_cast<uint2*>(out) = f32x4_to_bf16x4_bits(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
  }
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

// Launches kernel i of the backward and returns the launch's own status; with
// timing events, its start and stop timestamps are taken from the dispatch itself
// (no extra packets in the stream).
struct Launcher {
  const hipEvent_t* ev;
  hipStream_t s;
  template <typename... KA, typename... A>
  hipError_t operator()(int i, void (*kernel)(KA...), dim3 grid, dim3 block, A... args) const {
    return launch_kernel_timed(kernel, grid, block, s, ev ? ev[2 * i] : nullptr, ev ? ev[2 * i + 1] : nullptr,
                               args...);
  }
  // a kernel that this path does not need: both marks back to back
  hipError_t skip(int i) const {
    hipError_t e = hipSuccess;
    if (ev && ev[2 * i]) e = hipEventRecord(ev[2 * i], s);
    if (e == hipSuccess && ev && ev[2 * i + 1]) e = hipEventRecord(ev[2 * i + 1], s);
    return e;
  }
};

// The three launches in order; the first one the runtime rejects ends the sequence,
// so no later kernel reads a workspace that an earlier one did not fill.
template <int D, int G>
hipError_t launch_bf16(const BwdArgs& a, const Launcher& run) {
  // Query heads per dQ work-group.  With 4 or more per KV head, work-groups of two
  // heads (each gathering the unit's tiles; the repeats mostly hit the XCD's L2) fit
  // two to a compute unit, so one's start-up overlaps the other's tiles.
  constexpr int HPW = G >= 4 ? 2 : G;
  hipError_t e = run(0, attend_bwd_dq_bf16_kernel<D, G, HPW>, dim3(xcd_grid(a.n_units * (G / HPW))),
                     dim3(128 * HPW), a);
  if (e == hipSuccess) e = run(1, attend_bwd_dkdv_bf16_kernel<D, G>, dim3(a.n_units * kMaxParts), dim3(256), a);
  if (e == hipSuccess)
    e = run(2, attend_bwd_dkdv_finalize_kernel<D>, dim3(a.n_units * kFinalizeSlices), dim3(256), a);
  return e;
}
template <int D>
hipError_t launch_bf16_g(const BwdArgs& a, int G, const Launcher& run) {
  switch (G) {
    case 1: return launch_bf16<D, 1>(a, run);
    case 2: return launch_bf16<D, 2>(a, run);
    case 4: return launch_bf16<D, 4>(a, run);
    default: return launch_bf16<D, 8>(a, run);
  }
}

}  // namespace

size_t bwd_workspace_bytes(const Dims& d) {
  // rowsum(dO*O) and -LSE log2(e) per query row, one flag per (sequence, KV head, active chunk), and
  // G fp32 dK/dV partials per active chunk (bf16 path only).
  const size_t rows = (size_t)d.B * d.Hq * (size_t)d.seg_len;
  const size_t units = (size_t)d.B * d.Hkv * (size_t)d.nb;
  const size_t parts = units * (size_t)kMaxParts * 2 * 64 * (size_t)d.D * sizeof(float);
  return DkdvLayout::part_off(rows, units, (size_t)d.nb) + parts;
}

hipError_t launch_attend_bwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* d_o,
                             const int32_t* group_idx, void* dq, void* dk, void* dv,
                             void* workspace, hipStream_t s, const hipEvent_t* events) {
  const Launcher run{events, s};
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.d_o = d_o; a.lse = lse; a.gidx = group_idx;
  a.dq = dq; a.dk = dk; a.dv = dv;
  {
    const size_t rows = (size_t)d.B * d.Hq * (size_t)d.seg_len;
    const size_t units = (size_t)d.B * d.Hkv * (size_t)d.nb;
    a.cls_count = (int*)workspace;
    a.dvec = (float*)((char*)workspace + DkdvLayout::dvec_off);
    a.nlse = (float*)((char*)workspace + DkdvLayout::nlse_off(rows));
    a.flags = (int*)((char*)workspace + DkdvLayout::flags_off(rows));
    a.vis = (int*)((char*)workspace + DkdvLayout::vis_off(rows, units));
    a.cls_items = (int4*)((char*)workspace + DkdvLayout::items_off(rows, units, (size_t)d.nb));
    a.parts = (float*)((char*)workspace + DkdvLayout::part_off(rows, units, (size_t)d.nb));
  }
  a.t_cap = d.t_cap; a.t_hist = d.t_hist; a.seg_len = d.seg_len;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.kg = d.kg; a.nb = d.nb; a.n_units = d.B * d.Hkv * d.nb;
  a.scale = d.scale;
  a.target_rounds = d.t_hist >= 3 * d.seg_len ? kTargetRoundsLongHistory : kTargetRoundsShortHistory;
  const int grid = xcd_grid(a.n_units);
  if (bf16) return d.D == 128 ? launch_bf16_g<128>(a, d.G, run) : launch_bf16_g<64>(a, d.G, run);
  // fp32: dQ and dK/dV each in one kernel, no work list and no partial sums (the
  // class counts at the workspace start are not touched)
  hipError_t e = d.D == 128 ? run(0, attend_bwd_dq_f32_kernel<128>, dim3(grid), dim3(64 * d.G), a, d.G)
                            : run(0, attend_bwd_dq_f32_kernel<64>, dim3(grid), dim3(64 * d.G), a, d.G);
  if (e == hipSuccess)
    e = d.D == 128 ? run(1, attend_bwd_dkdv_f32_kernel<128>, dim3(grid), dim3(256), a, d.G)
                   : run(1, attend_bwd_dkdv_f32_kernel<64>, dim3(grid), dim3(256), a, d.G);
  if (e == hipSuccess) e = run.skip(2);
  return e;
}

}  // namespace hga
