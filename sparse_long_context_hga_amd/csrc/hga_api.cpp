// C ABI of the HGA routed-attention library: host-side argument validation and
// kernel dispatch.  Every check runs before anything is enqueued, so a rejected
// call has no effect on the device.
#include "hga.h"
#include "hga_internal.h"

#include <math.h>

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the static shape and the positions, fills `d`.  need_seg: seg_len must be > 0.
int resolve(const hga_shape* s, int64_t t_cap, int64_t t_hist, int64_t seg_len, hga::Dims& d) {
  if (!s) return HGA_ERR_NULL;
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads != 0)
    return HGA_ERR_SHAPE;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HGA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return HGA_ERR_UNSUPPORTED;
  if (s->chunk != 64 || s->group != 8 || s->q_block != 64) return HGA_ERR_UNSUPPORTED;
  if (s->dtype != HGA_F32 && s->dtype != HGA_BF16) return HGA_ERR_UNSUPPORTED;
  if (s->top_chunks < 0 || s->top_groups < 0) return HGA_ERR_SHAPE;
  if (s->top_chunks > 64) return HGA_ERR_UNSUPPORTED;
  if (s->top_groups > 8 * s->top_chunks) return HGA_ERR_SHAPE;
  if (!isfinite(s->softmax_scale)) return HGA_ERR_SHAPE;
  if (t_cap <= 0 || t_cap % 64 != 0) return HGA_ERR_SHAPE;
  if (t_hist < 0 || t_hist % 64 != 0 || seg_len < 0 || seg_len % 64 != 0) return HGA_ERR_SHAPE;
  if (t_hist + seg_len > t_cap) return HGA_ERR_CAPACITY;
  // unit counts are 32-bit on the device
  if ((int64_t)s->batch * s->n_kv_heads * (seg_len / 64 + 1) > (int64_t)1 << 30) return HGA_ERR_UNSUPPORTED;
  d.B = s->batch;
  d.Hq = s->n_q_heads;
  d.Hkv = s->n_kv_heads;
  d.G = G;
  d.D = s->head_dim;
  d.kc = s->top_chunks;
  d.kg = s->top_groups;
  d.t_cap = t_cap;
  d.t_hist = t_hist;
  d.seg_len = seg_len;
  d.nb = (int)(seg_len / 64);
  d.scale = s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
  return HGA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? HGA_OK : HGA_ERR_HIP; }

}  // namespace

extern "C" {

int hga_build_summaries(const hga_shape* shape, const void* k_cache, int64_t t_cap, int64_t t_begin,
                        int64_t t_end, void* group_sum, void* chunk_sum, void* stream) {
  hga::Dims d;
  if (t_begin < 0 || t_end < t_begin || t_begin % 64 != 0 || t_end % 64 != 0) {
    if (!shape) return HGA_ERR_NULL;
    return HGA_ERR_SHAPE;
  }
  int st = resolve(shape, t_cap, t_begin, t_end - t_begin, d);
  if (st != HGA_OK) return st;
  if (t_end == t_begin) return HGA_OK;
  if (!k_cache || !group_sum || !chunk_sum) return HGA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(group_sum) || !aligned16(chunk_sum)) return HGA_ERR_ALIGN;
  return hip_status(hga::launch_summaries(d, shape->dtype == HGA_BF16, k_cache, t_begin, t_end, group_sum,
                                          chunk_sum, (hipStream_t)stream));
}

static int route_impl(const hga_shape* shape, const void* q, const void* q_prev, bool causal,
                      const void* chunk_sum, const void* group_sum, int64_t t_cap, int64_t t_hist,
                      int64_t seg_len, int32_t* chunk_idx, int32_t* group_idx, float* chunk_score,
                      float* group_score, void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, t_hist, seg_len, d);
  if (st != HGA_OK) return st;
  if (seg_len == 0) return HGA_ERR_SHAPE;
  if ((t_hist + seg_len) / 64 > HGA_MAX_CHUNKS) return HGA_ERR_UNSUPPORTED;
  if (!q || !chunk_sum || !group_sum || (d.kc > 0 && !chunk_idx) || (d.kg > 0 && !group_idx))
    return HGA_ERR_NULL;
  if (causal && t_hist > 0 && !q_prev) return HGA_ERR_NULL;
  if (!aligned16(q) || !aligned16(chunk_sum) || !aligned16(group_sum) ||
      (chunk_idx && !aligned16(chunk_idx)) || (group_idx && !aligned16(group_idx)) ||
      (chunk_score && !aligned16(chunk_score)) ||
      (group_score && !aligned16(group_score)) || (causal && q_prev && !aligned16(q_prev)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_route(d, shape->dtype == HGA_BF16, q, causal ? q_prev : nullptr, causal,
                                      chunk_sum, group_sum, chunk_idx, group_idx, chunk_score, group_score,
                                      (hipStream_t)stream));
}

int hga_route(const hga_shape* shape, const void* q, const void* chunk_sum, const void* group_sum,
              int64_t t_cap, int64_t t_hist, int64_t seg_len, int32_t* chunk_idx, int32_t* group_idx,
              float* chunk_score, float* group_score, void* stream) {
  return route_impl(shape, q, nullptr, false, chunk_sum, group_sum, t_cap, t_hist, seg_len, chunk_idx,
                    group_idx, chunk_score, group_score, stream);
}

int hga_route_causal(const hga_shape* shape, const void* q, const void* q_prev, const void* chunk_sum,
                     const void* group_sum, int64_t t_cap, int64_t t_hist, int64_t seg_len,
                     int32_t* chunk_idx, int32_t* group_idx, float* chunk_score, float* group_score,
                     void* stream) {
  return route_impl(shape, q, q_prev, true, chunk_sum, group_sum, t_cap, t_hist, seg_len, chunk_idx,
                    group_idx, chunk_score, group_score, stream);
}

int hga_attend_fwd(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                   int64_t t_cap, int64_t t_hist, int64_t seg_len, const int32_t* group_idx, void* o,
                   float* lse, void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, t_hist, seg_len, d);
  if (st != HGA_OK) return st;
  if (seg_len == 0) return HGA_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !o || !lse || (d.kg > 0 && !group_idx)) return HGA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      (group_idx && !aligned16(group_idx)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_attend_fwd(d, shape->dtype == HGA_BF16, q, k_cache, v_cache, group_idx, o,
                                           lse, (hipStream_t)stream));
}

static int forward_impl(const hga_shape* shape, const void* q, const void* q_prev, bool causal, const void* k_cache,
                        const void* v_cache, void* chunk_sum, void* group_sum, int64_t t_cap, int64_t t_hist,
                        int64_t seg_len, int32_t* chunk_idx, int32_t* group_idx, void* o, float* lse,
                        void* const* events, void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, t_hist, seg_len, d);
  if (st != HGA_OK) return st;
  if (seg_len == 0) return HGA_ERR_SHAPE;
  if ((t_hist + seg_len) / 64 > HGA_MAX_CHUNKS) return HGA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !chunk_sum || !group_sum || !o || !lse || (d.kc > 0 && !chunk_idx) ||
      (d.kg > 0 && !group_idx))
    return HGA_ERR_NULL;
  if (causal && t_hist > 0 && !q_prev) return HGA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(chunk_sum) ||
      !aligned16(group_sum) || !aligned16(o) || !aligned16(lse) || (chunk_idx && !aligned16(chunk_idx)) ||
      (group_idx && !aligned16(group_idx)) || (causal && q_prev && !aligned16(q_prev)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_forward(d, shape->dtype == HGA_BF16, q, causal ? q_prev : nullptr, causal, k_cache,
                                        v_cache, chunk_sum, group_sum, chunk_idx, group_idx, o, lse,
                                        (hipStream_t)stream, (const hipEvent_t*)events));
}

int hga_forward(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache, void* chunk_sum,
                void* group_sum, int64_t t_cap, int64_t t_hist, int64_t seg_len, int32_t* chunk_idx,
                int32_t* group_idx, void* o, float* lse, void* const* events, void* stream) {
  return forward_impl(shape, q, nullptr, false, k_cache, v_cache, chunk_sum, group_sum, t_cap, t_hist, seg_len,
                      chunk_idx, group_idx, o, lse, events, stream);
}

int hga_forward_causal(const hga_shape* shape, const void* q, const void* q_prev, const void* k_cache,
                       const void* v_cache, void* chunk_sum, void* group_sum, int64_t t_cap, int64_t t_hist,
                       int64_t seg_len, int32_t* chunk_idx, int32_t* group_idx, void* o, float* lse,
                       void* const* events, void* stream) {
  return forward_impl(shape, q, q_prev, true, k_cache, v_cache, chunk_sum, group_sum, t_cap, t_hist, seg_len,
                      chunk_idx, group_idx, o, lse, events, stream);
}

int64_t hga_stage_history_min(const hga_shape* shape, int64_t t_hist, int64_t seg_len) {
  hga::Dims d;
  if (resolve(shape, t_hist + seg_len > 0 ? t_hist + seg_len : 64, t_hist, seg_len, d) != HGA_OK) return -1;
  const int64_t sel = (int64_t)8 * d.nb * d.kg;                 // at most this many selected history tokens
  const int64_t need = t_hist < sel ? t_hist : sel;
  return (need + 63) / 64 * 64;
}

int hga_stage_history(const hga_shape* shape, const void* k_host, const void* v_host, int64_t host_t_cap,
                      int64_t t_hist, int64_t seg_len, const int32_t* group_idx, void* k_stage, void* v_stage,
                      int64_t stage_cap, int64_t stage_hist, int32_t* group_idx_stage, void* stream) {
  // (k_host / v_host: pinned host memory; the kernel reads it through its device mapping)
  hga::Dims d;
  int st = resolve(shape, t_hist + seg_len > 0 ? t_hist + seg_len : 64, t_hist, seg_len, d);
  if (st != HGA_OK) return st;
  if (seg_len == 0) return HGA_ERR_SHAPE;
  if (host_t_cap < t_hist || host_t_cap % 64 != 0 || stage_cap % 64 != 0 || stage_hist % 64 != 0 ||
      stage_hist < 0)
    return HGA_ERR_SHAPE;
  if (t_hist / 8 > (int64_t)HGA_MAX_CHUNKS * 8 || (t_hist + seg_len) / 64 > HGA_MAX_CHUNKS)
    return HGA_ERR_UNSUPPORTED;
  if (stage_hist < hga_stage_history_min(shape, t_hist, seg_len) || stage_hist + seg_len > stage_cap)
    return HGA_ERR_CAPACITY;
  if (d.kg == 0) return HGA_OK;   // nothing selected, nothing to stage or renumber
  if (!k_host || !v_host || !group_idx || !k_stage || !v_stage || !group_idx_stage) return HGA_ERR_NULL;
  if (!aligned16(k_host) || !aligned16(v_host) || !aligned16(group_idx) || !aligned16(k_stage) ||
      !aligned16(v_stage) || !aligned16(group_idx_stage))
    return HGA_ERR_ALIGN;
  void* kd = nullptr;
  void* vd = nullptr;
  if (hipHostGetDevicePointer(&kd, const_cast<void*>(k_host), 0) != hipSuccess ||
      hipHostGetDevicePointer(&vd, const_cast<void*>(v_host), 0) != hipSuccess)
    return HGA_ERR_UNSUPPORTED;   // not pinned host memory
  return hip_status(hga::launch_stage_history(d, shape->dtype == HGA_BF16, kd, vd, host_t_cap, group_idx, k_stage,
                                              v_stage, stage_cap, stage_hist, group_idx_stage,
                                              (hipStream_t)stream));
}

size_t hga_attend_bwd_workspace_size(const hga_shape* shape, int64_t t_hist, int64_t seg_len) {
  hga::Dims d;
  if (resolve(shape, t_hist + seg_len > 0 ? t_hist + seg_len : 64, t_hist, seg_len, d) != HGA_OK) return 0;
  return hga::bwd_workspace_bytes(d);
}

static int attend_bwd_impl(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                   const void* o, const float* lse, const void* d_o, int64_t t_cap, int64_t t_hist,
                   int64_t seg_len, const int32_t* group_idx, void* dq, void* dk_active, void* dv_active,
                   void* workspace, size_t workspace_bytes, void* const* events, void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, t_hist, seg_len, d);
  if (st != HGA_OK) return st;
  if (seg_len == 0) return HGA_ERR_SHAPE;
  if (seg_len / 64 > 1024) return HGA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !o || !lse || !d_o || !dq || !dk_active || !dv_active ||
      (d.kg > 0 && !group_idx))
    return HGA_ERR_NULL;
  if (!workspace || workspace_bytes < hga::bwd_workspace_bytes(d)) return HGA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(d_o) || !aligned16(dq) || !aligned16(dk_active) || !aligned16(dv_active) ||
      !aligned16(workspace) || (group_idx && !aligned16(group_idx)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_attend_bwd(d, shape->dtype == HGA_BF16, q, k_cache, v_cache, o, lse, d_o,
                                           group_idx, dq, dk_active, dv_active, workspace,
                                           (hipStream_t)stream, (const hipEvent_t*)events));
}

size_t hga_decode_workspace_size(const hga_shape* shape, int64_t t_cap) {
  hga::Dims d;
  if (resolve(shape, t_cap, 0, 0, d) != HGA_OK) return 0;
  return hga::decode_workspace_bytes(d);
}

static int decode_ws_check(const hga::Dims& d, const void* workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < hga::decode_workspace_bytes(d)) return HGA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HGA_ERR_ALIGN;
  return HGA_OK;
}

int hga_decode_route(const hga_shape* shape, const void* q, const void* chunk_sum, const void* group_sum,
                     int64_t t_cap, const int32_t* pos, int32_t* chunk_idx, int32_t* group_idx,
                     float* chunk_score, float* group_score, void* workspace, size_t workspace_bytes,
                     void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, 0, 0, d);
  if (st != HGA_OK) return st;
  if (t_cap / 64 > HGA_MAX_CHUNKS) return HGA_ERR_UNSUPPORTED;
  if (!q || !chunk_sum || !group_sum || !pos || (d.kc > 0 && !chunk_idx) || (d.kg > 0 && !group_idx))
    return HGA_ERR_NULL;
  if ((st = decode_ws_check(d, workspace, workspace_bytes)) != HGA_OK) return st;
  if (!aligned16(q) || !aligned16(chunk_sum) || !aligned16(group_sum) ||
      (chunk_idx && !aligned16(chunk_idx)) || (group_idx && !aligned16(group_idx)) ||
      (chunk_score && !aligned16(chunk_score)) || (group_score && !aligned16(group_score)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_decode(d, shape->dtype == HGA_BF16, true, false, q, nullptr, nullptr, chunk_sum,
                                       group_sum, pos, chunk_idx, group_idx, chunk_score, group_score, nullptr,
                                       nullptr, nullptr, nullptr, workspace, (hipStream_t)stream));
}

int hga_decode_attend(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                      int64_t t_cap, const int32_t* pos, const int32_t* group_idx, void* o, float* lse,
                      void* group_sum, void* chunk_sum, void* workspace, size_t workspace_bytes, void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, 0, 0, d);
  if (st != HGA_OK) return st;
  if (!q || !k_cache || !v_cache || !pos || !o || !lse || (d.kg > 0 && !group_idx)) return HGA_ERR_NULL;
  if ((group_sum == nullptr) != (chunk_sum == nullptr)) return HGA_ERR_NULL;
  if ((st = decode_ws_check(d, workspace, workspace_bytes)) != HGA_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      (group_idx && !aligned16(group_idx)) || (group_sum && !aligned16(group_sum)) ||
      (chunk_sum && !aligned16(chunk_sum)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_decode(d, shape->dtype == HGA_BF16, false, true, q, k_cache, v_cache, nullptr,
                                       nullptr, pos, nullptr, const_cast<int32_t*>(group_idx), nullptr, nullptr,
                                       o, lse, group_sum, chunk_sum, workspace, (hipStream_t)stream));
}

int hga_decode_step(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                    void* chunk_sum, void* group_sum, int64_t t_cap, const int32_t* pos, int32_t* chunk_idx,
                    int32_t* group_idx, void* o, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, 0, 0, d);
  if (st != HGA_OK) return st;
  if (t_cap / 64 > HGA_MAX_CHUNKS) return HGA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !chunk_sum || !group_sum || !pos || !o || !lse || (d.kg > 0 && !group_idx))
    return HGA_ERR_NULL;
  if ((st = decode_ws_check(d, workspace, workspace_bytes)) != HGA_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(chunk_sum) || !aligned16(group_sum) || (chunk_idx && !aligned16(chunk_idx)) ||
      (group_idx && !aligned16(group_idx)))
    return HGA_ERR_ALIGN;
  return hip_status(hga::launch_decode(d, shape->dtype == HGA_BF16, true, true, q, k_cache, v_cache, chunk_sum,
                                       group_sum, pos, chunk_idx, group_idx, nullptr, nullptr, o, lse, group_sum,
                                       chunk_sum, workspace, (hipStream_t)stream));
}

int hga_decode_step_noalloc(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                            void* chunk_sum, void* group_sum, int64_t t_cap, const int32_t* pos,
                            int32_t* chunk_idx, int32_t* group_idx, void* o, float* lse, void* stream) {
  hga::Dims d;
  int st = resolve(shape, t_cap, 0, 0, d);
  if (st != HGA_OK) return st;
  if (t_cap / 64 > HGA_MAX_CHUNKS) return HGA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !chunk_sum || !group_sum || !pos || !o || !lse || (d.kg > 0 && !group_idx))
    return HGA_ERR_NULL;
  static_assert(hga::kNoallocScratchBytes == (size_t)HGA_DECODE_NOALLOC_MAX_BYTES, "header and library agree");
  static_assert(hga::kNoallocCounterSlots == (size_t)HGA_DECODE_NOALLOC_MAX_UNITS, "header and library agree");
  if ((size_t)d.B * d.Hkv > hga::kNoallocCounterSlots ||
      hga::decode_workspace_bytes(d, hga::kNoallocCounterSlots) > hga::kNoallocScratchBytes)
    return HGA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(chunk_sum) || !aligned16(group_sum) || (chunk_idx && !aligned16(chunk_idx)) ||
      (group_idx && !aligned16(group_idx)))
    return HGA_ERR_ALIGN;
  void* ws = nullptr;
  if (hga::noalloc_scratch(&ws, (hipStream_t)stream) != hipSuccess) return HGA_ERR_HIP;
  return hip_status(hga::launch_decode(d, shape->dtype == HGA_BF16, true, true, q, k_cache, v_cache, chunk_sum,
                                       group_sum, pos, chunk_idx, group_idx, nullptr, nullptr, o, lse, group_sum,
                                       chunk_sum, ws, (hipStream_t)stream, hga::kNoallocCounterSlots));
}

int hga_attend_bwd(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                   const void* o, const float* lse, const void* d_o, int64_t t_cap, int64_t t_hist,
                   int64_t seg_len, const int32_t* group_idx, void* dq, void* dk_active, void* dv_active,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return attend_bwd_impl(shape, q, k_cache, v_cache, o, lse, d_o, t_cap, t_hist, seg_len, group_idx, dq,
                         dk_active, dv_active, workspace, workspace_bytes, nullptr, stream);
}

int hga_attend_bwd_timed(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                         const void* o, const float* lse, const void* d_o, int64_t t_cap, int64_t t_hist,
                         int64_t seg_len, const int32_t* group_idx, void* dq, void* dk_active,
                         void* dv_active, void* workspace, size_t workspace_bytes, void* const* events,
                         void* stream) {
  if (!events) return HGA_ERR_NULL;
  return attend_bwd_impl(shape, q, k_cache, v_cache, o, lse, d_o, t_cap, t_hist, seg_len, group_idx, dq,
                         dk_active, dv_active, workspace, workspace_bytes, events, stream);
}

const char* hga_status_string(int status) {
  switch (status) {
    case HGA_OK: return "ok";
    case HGA_ERR_NULL: return "a required pointer is NULL";
    case HGA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case HGA_ERR_UNSUPPORTED: return "unsupported configuration";
    case HGA_ERR_CAPACITY: return "positions exceed the cache capacity t_cap";
    case HGA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case HGA_ERR_WORKSPACE: return "workspace missing or too small";
    case HGA_ERR_HIP: return "the HIP runtime rejected a launch";
    default: return "unknown status";
  }
}

}  // extern "C"
