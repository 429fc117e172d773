// Host-side launch interface between the C ABI (hga_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hga {

// Validated, resolved sizes of one call.
struct Dims {
  int B, Hq, Hkv, G, D;
  int kc, kg;
  int64_t t_cap, t_hist, seg_len;
  int nb;        // query blocks in the active segment (seg_len / 64)
  float scale;   // softmax scale
};

hipError_t launch_summaries(const Dims& d, bool bf16, const void* k, int64_t t_begin, int64_t t_end,
                            void* group_sum, void* chunk_sum, hipStream_t s);

// causal: block j is routed by the rows of block j-1 (q_prev [B,Hq,64,d] for j = 0).
hipError_t launch_route(const Dims& d, bool bf16, const void* q, const void* q_prev, bool causal,
                        const void* chunk_sum, const void* group_sum, int32_t* chunk_idx,
                        int32_t* group_idx, float* chunk_score, float* group_score, hipStream_t s);

hipError_t launch_attend_fwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const int32_t* group_idx, void* o, float* lse, hipStream_t s);

// Workspace: one float per query row (rowsum(dO * O)).
size_t bwd_workspace_bytes(const Dims& d);

hipError_t launch_attend_bwd(const Dims& d, bool bf16, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* d_o,
                             const int32_t* group_idx, void* dq, void* dk, void* dv,
                             void* workspace, hipStream_t s, const hipEvent_t* events = nullptr);

// Generation path (one token per sequence; pos [B] on the device): routing,
// attention, or both (two launches); ws: decode_workspace_bytes(d) bytes.
size_t decode_workspace_bytes(const Dims& d);
hipError_t launch_decode(const Dims& d, bool bf16, bool route, bool attend, const void* q, const void* k,
                         const void* v, const void* chunk_sum, const void* group_sum, const int32_t* pos,
                         int32_t* chunk_idx, int32_t* group_idx, float* chunk_score, float* group_score,
                         void* o, float* lse, void* group_sum_out, void* chunk_sum_out, void* ws,
                         hipStream_t s);

}  // namespace hga
