// Host-side launch interface between the C ABI (hga_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hga {

template <typename T>
struct no_deduce { using type = T; };

// Launch of kernel `k` on stream `s` that returns this launch's own status: the
// HIP launch call reports it directly, so an error left behind by an unrelated
// earlier HIP call on the thread is neither returned nor cleared.  With start /
// stop events (may be null) the dispatch itself records them.
template <typename... P>
hipError_t launch_kernel_timed(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                               hipEvent_t stop, typename no_deduce<P>::type... args) {
  void* ptrs[] = {static_cast<void*>(&args)...};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, s, start, stop, 0);
}
template <typename... P>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s,
                         typename no_deduce<P>::type... args) {
  return launch_kernel_timed(k, grid, block, s, nullptr, nullptr, args...);
}

// Validated, resolved sizes of one call.
struct Dims {
  int B, Hq, Hkv, G, D;
  int kc, kg;
  int64_t t_cap, t_hist, seg_len;
  int nb;        // query blocks in the active segment (seg_len / 64)
  float scale;   // softmax scale
};

// Optional start / stop events are recorded by the dispatches themselves.
hipError_t launch_summaries(const Dims& d, bool bf16, const void* k, int64_t t_begin, int64_t t_end,
                            void* group_sum, void* chunk_sum, hipStream_t s, hipEvent_t start = nullptr,
                            hipEvent_t stop = nullptr);

// causal: block j is routed by the rows of block j-1 (q_prev [B,Hq,64,d] for j = 0).
hipError_t launch_route(const Dims& d, bool bf16, const void* q, const void* q_prev, bool causal,
                        const void* chunk_sum, const void* group_sum, int32_t* chunk_idx,
                        int32_t* group_idx, float* chunk_score, float* group_score, hipStream_t s,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

hipError_t launch_attend_fwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const int32_t* group_idx, void* o, float* lse, hipStream_t s, hipEvent_t start = nullptr,
                             hipEvent_t stop = nullptr);

// The forward of a segment: summaries of the active segment [t_hist, t_hist +
// seg_len), then routing (by each block's own rows, or with causal by the block
// before it, q_prev for the first) and attention: one kernel that does both per unit
// for bf16 with 4 query heads per KV head, else the route and attention kernels.
// ev: null, or 4 events: [0], [1] around the summaries, [2] at the start of the
// routing and [3] at the end of the attention.
hipError_t launch_forward(const Dims& d, bool bf16, const void* q, const void* q_prev, bool causal, const void* k,
                          const void* v, void* chunk_sum, void* group_sum, int32_t* chunk_idx, int32_t* group_idx,
                          void* o, float* lse, hipStream_t s, const hipEvent_t* ev);

// Host-RAM history tier: the selected history groups of every (sequence, KV head)
// copied from host memory into a staging cache, and the selection renumbered for it.
hipError_t launch_stage_history(const Dims& d, bool bf16, const void* k_host, const void* v_host, int64_t host_t_cap,
                                const int32_t* group_idx, void* k_stage, void* v_stage, int64_t stage_cap,
                                int64_t stage_hist, int32_t* group_idx_stage, hipStream_t s);

// Workspace: one float per query row (rowsum(dO * O)).
size_t bwd_workspace_bytes(const Dims& d);

hipError_t launch_attend_bwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* d_o,
                             const int32_t* group_idx, void* dq, void* dk, void* dv,
                             void* workspace, hipStream_t s, const hipEvent_t* events = nullptr);

// Generation path (one token per sequence; pos [B] on the device): routing,
// attention, or both (two launches); ws: decode_workspace_bytes(d) bytes.  The
// workspace starts with two arrays of arrival counters, counter_slots entries each
// (at least one per (sequence, KV head) unit; 0 means exactly one per unit), that
// must be zero before the first call and that every call leaves at zero.
size_t decode_workspace_bytes(const Dims& d, size_t counter_slots = 0);
// Bytes of the two counter arrays at the start of such a workspace.
size_t decode_counter_bytes(size_t counter_slots);

// The entry point that allocates nothing takes the generation step's workspace from
// a static device array of this size, laid out with this many counter slots.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
constexpr size_t kNoallocCounterSlots = (size_t)1 << 14;
// Device address of the current device's array (looked up once per device).
hipError_t noalloc_scratch(void** ptr, hipStream_t s);
hipError_t launch_decode(const Dims& d, bool bf16, bool route, bool attend, const void* q, const void* k,
                         const void* v, const void* chunk_sum, const void* group_sum, const int32_t* pos,
                         int32_t* chunk_idx, int32_t* group_idx, float* chunk_score, float* group_score,
                         void* o, float* lse, void* group_sum_out, void* chunk_sum_out, void* ws,
                         hipStream_t s, size_t counter_slots = 0);

}  // namespace hga
