// Host-RAM history tier: the detached history's K/V live in pinned host memory,
// and a segment's attention needs only the groups that its query blocks selected
// (the history is offloaded to RAM or NVMe on the pages: adnankhan.ai note, "Raw
// Abstract / Excerpt"; seventnews, "HGA的不同之处").  After routing (over summaries
// that stay in HBM), this kernel copies the selected history groups of every
// (sequence, KV head) from host memory into a compact staging cache in HBM and
// renumbers the selection for it, so that the attention kernels run unchanged on
// the staging cache.
//
// Staging layout per (sequence, KV head): slot s holds the s-th distinct selected
// history group (ascending ids), tokens 8s .. 8s+7; the active segment follows at
// stage_hist.  Renumbering keeps every selection ascending and every tile's groups
// in the same order, so attention over the staging cache is bit-identical to
// attention over the full cache.
//
// One launch of (sequences x KV heads) x kStageParts work-groups.  Every work-group
// of a (sequence, KV head) marks the selected history groups in an LDS bitmap (one
// bit per history group), turns it into slot numbers with a prefix count of the
// bitmap words, and copies the groups of the slots s with s % kStageParts equal to
// its part (a wave per group: each lane moves 16-byte pieces of the group's 8 rows
// of K and of V over the host link); part 0 also writes the renumbered selection.
#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kStageThreads = 256;
constexpr int kStageParts = 32;                       // work-groups per (sequence, KV head)
constexpr int kMaxHistGroups = 8192 * 8;             // one bitmap bit per history group (HGA_MAX_CHUNKS chunks)
constexpr int kBitmapWords = kMaxHistGroups / 32;
constexpr int kWordsPerThread = kBitmapWords / kStageThreads;

struct StageArgs {
  const uint16_t* k_host;   // [B, Hkv, host_t_cap, D] bytes as 16-bit words (element size irrelevant)
  const uint16_t* v_host;
  const int32_t* gidx;      // [B, Hkv, nb, kg]
  uint16_t* k_stage;        // [B, Hkv, stage_cap, D]
  uint16_t* v_stage;
  int32_t* gidx_stage;      // [B, Hkv, nb, kg]
  int64_t host_t_cap, stage_cap;
  int n_hist_groups;        // t_hist / 8
  int stage_groups;         // stage_hist / 8: renumbering of the active segment's groups
  int n_ids;                // nb * kg
  int row_bytes;            // D * element size
};

__global__ __launch_bounds__(kStageThreads) void stage_history_kernel(StageArgs a) {
  __shared__ uint32_t bits[kBitmapWords];
  __shared__ int base[kBitmapWords];   // selected groups in the words before
  __shared__ int scan_sh[kStageThreads / 64];
  __shared__ int list[kMaxHistGroups / kStageParts + 1];
  __shared__ int n_list;
  const int bh = blockIdx.x / kStageParts, part = blockIdx.x % kStageParts;
  const int tid = threadIdx.x;
  const int n_words = (a.n_hist_groups + 31) / 32;
  for (int i = tid; i < n_words; i += kStageThreads) bits[i] = 0u;
  if (tid == 0) n_list = 0;
  __syncthreads();
  const int32_t* g = a.gidx + (int64_t)bh * a.n_ids;
  for (int i = tid; i < a.n_ids; i += kStageThreads) {
    const int id = g[i];
    if (id >= 0 && id < a.n_hist_groups) atomicOr(&bits[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  // prefix count of the words: thread t owns words t*W .. t*W+W-1
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kWordsPerThread; ++k) {
    const int wi = tid * kWordsPerThread + k;
    cnt += wi < n_words ? __popc(bits[wi]) : 0;
  }
  int total;
  int run = block_exclusive_scan<kStageThreads>(cnt, scan_sh, total);
#pragma unroll
  for (int k = 0; k < kWordsPerThread; ++k) {
    const int wi = tid * kWordsPerThread + k;
    if (wi < n_words) {
      base[wi] = run;
      run += __popc(bits[wi]);
    }
  }
  __syncthreads();
  auto slot_of = [&](int id) __attribute__((always_inline)) {
    const uint32_t w = bits[id >> 5];
    return base[id >> 5] + __popc(w & ((1u << (id & 31)) - 1u));
  };
  if (part == 0) {   // the renumbered selection
    int32_t* out = a.gidx_stage + (int64_t)bh * a.n_ids;
    for (int i = tid; i < a.n_ids; i += kStageThreads) {
      const int id = g[i];
      out[i] = id < 0 ? -1 : id < a.n_hist_groups ? slot_of(id) : a.stage_groups + (id - a.n_hist_groups);
    }
  }
  // this part's groups: slots s with s % kStageParts == part, listed by s / kStageParts
#pragma unroll
  for (int k = 0; k < kWordsPerThread; ++k) {
    const int wi = tid * kWordsPerThread + k;
    if (wi < n_words) {
      uint32_t w = bits[wi];
      int s = base[wi];
      while (w) {
        const int bit = __ffs(w) - 1;
        w &= w - 1u;
        if (s % kStageParts == part) list[s / kStageParts] = wi * 32 + bit;
        ++s;
      }
    }
  }
  if (tid == 0) n_list = (total - part + kStageParts - 1) / kStageParts;
  __syncthreads();
  // copies: a wave per group, 8 rows of K then of V, 16 bytes per lane per step
  const int wave = tid >> 6, lane = tid & 63;
  const int group_bytes = 8 * a.row_bytes;            // contiguous in both caches
  const int64_t host_bh = (int64_t)bh * a.host_t_cap * a.row_bytes;
  const int64_t stage_bh = (int64_t)bh * a.stage_cap * a.row_bytes;
  for (int i = wave; i < n_list; i += kStageThreads / 64) {
    const int id = list[i];
    const int s = i * kStageParts + part;
    const char* hk = (const char*)a.k_host + host_bh + (int64_t)id * group_bytes;
    const char* hv = (const char*)a.v_host + host_bh + (int64_t)id * group_bytes;
    char* sk = (char*)a.k_stage + stage_bh + (int64_t)s * group_bytes;
    char* sv = (char*)a.v_stage + stage_bh + (int64_t)s * group_bytes;
    for (int off = lane * 16; off < group_bytes; off += 64 * 16) {
      const uint4 xk = *reinterpret_cast<const uint4*>(hk + off);
      const uint4 xv = *reinterpret_cast<const uint4*>(hv + off);
      *reinterpret_cast<uint4*>(sk + off) = xk;
      *reinterpret_cast<uint4*>(sv + off) = xv;
    }
  }
}

}  // namespace

hipError_t launch_stage_history(const Dims& d, bool bf16, const void* k_host, const void* v_host, int64_t host_t_cap,
                                const int32_t* group_idx, void* k_stage, void* v_stage, int64_t stage_cap,
                                int64_t stage_hist, int32_t* group_idx_stage, hipStream_t s) {
  StageArgs a;
  a.k_host = (const uint16_t*)k_host; a.v_host = (const uint16_t*)v_host;
  a.gidx = group_idx; a.k_stage = (uint16_t*)k_stage; a.v_stage = (uint16_t*)v_stage;
  a.gidx_stage = group_idx_stage;
  a.host_t_cap = host_t_cap; a.stage_cap = stage_cap;
  a.n_hist_groups = (int)(d.t_hist / kGroup);
  a.stage_groups = (int)(stage_hist / kGroup);
  a.n_ids = d.nb * d.kg;
  a.row_bytes = d.D * (bf16 ? 2 : 4);
  const dim3 grid((unsigned)(d.B * d.Hkv * kStageParts));
  return launch_kernel(stage_history_kernel, grid, dim3(kStageThreads), s, a);
}

}  // namespace hga
