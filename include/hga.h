/*
 * hga.h -- C ABI of the Hierarchical Global Attention (HGA) routed-attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * Method (pages on "Long-Context Fine-Tuning with Limited VRAM", arXiv 2607.15105):
 * the causal history is cut into 64-token chunks, each kept as a compact
 * summary vector, with 8-token group summaries inside each chunk; a query block
 * scores the chunk summaries with its own projected queries (no learned router
 * weights), keeps the top-k chunks, opens them at group level, keeps the top
 * groups, and runs exact attention over the exact-token K/V of the selected
 * groups (seventnews article, section "HGA的不同之处").  Training is segment-wise:
 * only the active segment is differentiable, older K/V is detached (adnankhan.ai
 * note, section "Raw Abstract / Excerpt").
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronizes; every call only enqueues kernels
 *    on `stream` (a hipStream_t handle; NULL = the default stream) and returns.
 *    Scratch memory comes from the caller (workspace arguments), or for
 *    hga_decode_step_noalloc from a static device array inside the library.
 *  - Tensors are dense, row-major, 16-byte aligned.  Float tensors (q, k, v, o,
 *    d_o, summaries, gradients) all have the element type shape->dtype
 *    (HGA_F32: IEEE float32; HGA_BF16: bfloat16).  lse and the optional score
 *    outputs are always float32; index tensors are int32.
 *  - Cache layout: k_cache / v_cache are [batch, n_kv_heads, t_cap, head_dim].
 *    Detached history occupies positions [0, t_hist); the active segment
 *    occupies [t_hist, t_hist + seg_len).
 *  - Query head h uses KV head h / (n_q_heads / n_kv_heads); one routing
 *    decision is made per (sequence, KV head, 64-token query block) and shared
 *    by the query heads of that KV head.
 *  - Errors: every argument is checked on the host before anything is enqueued.
 *    On error the call returns a negative hga_status, enqueues nothing and
 *    leaves all outputs untouched.  HGA_ERR_HIP means a launch was rejected by
 *    the HIP runtime (outputs then undefined).
 *  - Calls are re-entrant and thread-safe; the library holds no mutable state,
 *    except hga_decode_step_noalloc's static device scratch (see there).
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HGA_OK = 0,
  HGA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  HGA_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes                 */
  HGA_ERR_UNSUPPORTED = -3, /* valid but unsupported configuration                */
  HGA_ERR_CAPACITY = -4,    /* positions beyond t_cap                             */
  HGA_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                   */
  HGA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required         */
  HGA_ERR_HIP = -7          /* the HIP runtime rejected a launch                  */
} hga_status;

typedef enum { HGA_F32 = 0, HGA_BF16 = 1 } hga_dtype;

typedef struct {
  int32_t batch;        /* B >= 1                                                  */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads, Hq / Hkv in {1,2,4,8}      */
  int32_t n_kv_heads;   /* Hkv >= 1                                                */
  int32_t head_dim;     /* d in {64, 128}                                          */
  int32_t chunk;        /* chunk length; must be 64                                */
  int32_t group;        /* group length; must be 8                                 */
  int32_t q_block;      /* query-block length; must be 64 (= chunk, aligned)       */
  int32_t top_chunks;   /* k_c in [0, 64]: chunks kept per query block             */
  int32_t top_groups;   /* k_g in [0, 8*k_c]: groups kept among the selected chunks */
  int32_t dtype;        /* hga_dtype                                               */
  float softmax_scale;  /* logits = softmax_scale * q.k; <= 0 means 1/sqrt(d)      */
} hga_shape;

/* Longest supported context in chunks (t_cap / 64) for routing. */
#define HGA_MAX_CHUNKS 8192

/*
 * hga_build_summaries -- group and chunk summaries of the keys in
 * [t_begin, t_end).  The pages describe a compact summary per 64-token chunk
 * and a summary cache for its 8-token groups (seventnews, "HGA的不同之处";
 * gist.science, "解决方案") without a formula; this library defines the summary
 * as the mean of the keys, summed in fp32 in the fixed pairwise order
 *   group sum  g = ((k0+k1)+(k2+k3)) + ((k4+k5)+(k6+k7))
 *   chunk sum  c = the same tree over the chunk's 8 unscaled group sums
 * and stores g/8 and c/64 in the key dtype (bf16: round to nearest even).
 *
 *   k_cache    [B, Hkv, t_cap, d]              read
 *   group_sum  [B, Hkv, t_cap/8, d]            rows t_begin/8 .. t_end/8-1 written
 *   chunk_sum  [B, Hkv, t_cap/64, d]           rows t_begin/64 .. t_end/64-1 written
 *   t_begin, t_end: multiples of 64 with 0 <= t_begin <= t_end <= t_cap.
 * Rows outside the range are not touched, so history summaries are built once
 * and each new segment only adds its own rows.
 */
int hga_build_summaries(const hga_shape* shape, const void* k_cache, int64_t t_cap,
                        int64_t t_begin, int64_t t_end, void* group_sum, void* chunk_sum,
                        void* stream);

/*
 * hga_route -- two-level routing of every 64-token query block of the active
 * segment (seventnews, "HGA的不同之处": queries score the chunk summaries, keep
 * the top-k chunks, open them at group level; the router has no weights.
 * Block-level decisions from several positions: same article, "因果泄露").
 *
 * For block j (positions t_hist+64j .. +63) of sequence b and KV head g:
 *   rows       = the 64 positions x the Hq/Hkv query heads of KV head g
 *   candidates = chunks 0 .. J-1, J = t_hist/64 + j (every complete earlier chunk)
 *   sigma_c    = max over rows of (q . chunk_sum[c]), fp32
 *   chunks     = top min(k_c, J) by (sigma desc, index asc)
 *   groups     = the 8 groups of every selected chunk;
 *   tau_x      = max over rows of (q . group_sum[x]), fp32
 *   group_idx  = top min(k_g, #groups) by (tau desc, index asc)
 * Outputs are stored ascending and padded with -1:
 *   q          [B, Hq, seg_len, d]                       read
 *   chunk_sum  [B, Hkv, t_cap/64, d], group_sum [B, Hkv, t_cap/8, d]   read
 *   chunk_idx  [B, Hkv, seg_len/64, k_c] int32  (chunk ids)             written
 *   group_idx  [B, Hkv, seg_len/64, k_g] int32  (group ids; token = 8*id) written
 *   chunk_idx may be NULL when k_c == 0 and group_idx may be NULL when k_g == 0.
 *   chunk_score, group_score: optional (may be NULL) float32 arrays shaped like
 *   chunk_idx / group_idx holding sigma / tau of each selected id (-inf where
 *   the id is -1).
 * Requires seg_len > 0, t_hist and seg_len multiples of 64,
 * t_hist + seg_len <= t_cap, (t_hist + seg_len)/64 <= HGA_MAX_CHUNKS.
 */
int hga_route(const hga_shape* shape, const void* q, const void* chunk_sum,
              const void* group_sum, int64_t t_cap, int64_t t_hist, int64_t seg_len,
              int32_t* chunk_idx, int32_t* group_idx, float* chunk_score, float* group_score,
              void* stream);

/*
 * hga_route_causal -- strictly causal routing.  With hga_route a block's
 * decision reads all of its rows, so an earlier position can learn which chunks
 * its later positions favour (the side channel described in the seventnews
 * article, section "一个真正的警告：因果泄露", which names a strictly causal
 * variant as in development without giving one).  This library's variant routes
 * block j with the rows of the query block just before it, everything else as in
 * hga_route (candidates chunks 0 .. J-1, the group step, ties, output format):
 *   rows(j) = block j-1 of q                      for j >= 1
 *           = q_prev, the last 64-position block of the previous segment, for j = 0
 * Every input of the decision then lies before the block's first position.
 *   q_prev  [B, Hq, 64, d] read; required when t_hist > 0 (HGA_ERR_NULL if NULL),
 *           ignored when t_hist == 0 (the first block has no candidates).
 * Other arguments, requirements and errors as hga_route.  hga_attend_fwd and
 * hga_attend_bwd take the group_idx it writes unchanged.
 */
int hga_route_causal(const hga_shape* shape, const void* q, const void* q_prev,
                     const void* chunk_sum, const void* group_sum, int64_t t_cap, int64_t t_hist,
                     int64_t seg_len, int32_t* chunk_idx, int32_t* group_idx, float* chunk_score,
                     float* group_score, void* stream);

/*
 * hga_attend_fwd -- exact attention of every active query over the exact
 * tokens of its block's selected groups plus its own chunk up to and including
 * its own position (summaries never act as values: seventnews, "HGA的不同之处";
 * a bounded set of exact historical tokens per query block: the abstract).
 *
 *   q          [B, Hq, seg_len, d]                  read
 *   k_cache, v_cache [B, Hkv, t_cap, d]             read (only selected groups and
 *                                                   the active chunks are touched)
 *   group_idx  [B, Hkv, seg_len/64, k_g] int32      read; as written by hga_route
 *                                                   (ascending valid ids, then -1)
 *   o          [B, Hq, seg_len, d]                  written
 *   lse        [B, Hq, seg_len] float32             written: natural log of the sum
 *                                                   of exp(softmax_scale * q.k) over
 *                                                   the attended keys
 * group_idx is trusted: ids must be valid groups before the query block.  It may
 * be NULL when k_g == 0 (every query then attends its own chunk only).
 */
int hga_attend_fwd(const hga_shape* shape, const void* q, const void* k_cache,
                   const void* v_cache, int64_t t_cap, int64_t t_hist, int64_t seg_len,
                   const int32_t* group_idx, void* o, float* lse, void* stream);

/*
 * hga_forward -- the forward of one segment in one call: the summaries of the
 * active segment's chunks (as hga_build_summaries over [t_hist, t_hist + seg_len)),
 * then the routing of every query block (as hga_route) and the attention (as
 * hga_attend_fwd).  With bf16 and 4 query heads per KV head the routing and the
 * attention of a (sequence, KV head, query block) run in one work-group: the query
 * rows are read once for both, and the selection feeds the K/V gather from on-chip
 * memory; other shapes run the two kernels of hga_route and hga_attend_fwd.
 * Outputs equal those of the three separate calls (bit for bit).
 *
 *   q, k_cache, v_cache, t_cap, t_hist, seg_len: as hga_attend_fwd; the history's
 *              summaries (chunks below t_hist / 64) must already be built
 *   chunk_sum, group_sum: read, and written for the active segment's chunks
 *   chunk_idx, group_idx, o, lse: written, as hga_route and hga_attend_fwd
 *   events     NULL, or HGA_FWD_EVENTS hipEvent_t handles created by the caller
 *              (NULL entries skipped), recorded by the dispatches themselves:
 *              [0] / [1] at the start / end of the summaries kernel, [2] / [3] at
 *              the start of the routing and the end of the attention.
 * Requirements and errors as hga_route (chunk_idx and group_idx may not be NULL
 * while k_c resp. k_g is positive).
 */
#define HGA_FWD_EVENTS 4
int hga_forward(const hga_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                void* chunk_sum, void* group_sum, int64_t t_cap, int64_t t_hist, int64_t seg_len,
                int32_t* chunk_idx, int32_t* group_idx, void* o, float* lse, void* const* events,
                void* stream);

/*
 * hga_forward_causal -- hga_forward with strictly causal routing: the summaries of
 * the active segment, then the routing of every query block by the rows of the block
 * before it (as hga_route_causal; the side channel of block-level routing is the
 * subject of the seventnews article's section "一个真正的警告：因果泄露") and the
 * attention (as hga_attend_fwd).  With bf16 and 4 query heads per KV head a
 * (sequence, KV head, query block) is routed and attended in one work-group, which
 * reads the routing rows and then its own rows; other shapes run the two kernels.
 * Outputs equal those of hga_build_summaries, hga_route_causal and hga_attend_fwd
 * (bit for bit).
 *   q_prev  [B, Hq, 64, d] read, as hga_route_causal: required when t_hist > 0
 *           (HGA_ERR_NULL if NULL), ignored when t_hist == 0.
 * Other arguments, events, requirements and errors as hga_forward.
 */
int hga_forward_causal(const hga_shape* shape, const void* q, const void* q_prev, const void* k_cache,
                       const void* v_cache, void* chunk_sum, void* group_sum, int64_t t_cap, int64_t t_hist,
                       int64_t seg_len, int32_t* chunk_idx, int32_t* group_idx, void* o, float* lse,
                       void* const* events, void* stream);

/*
 * Host-RAM history tier.  The pages keep older K/V in RAM or on NVMe and bring
 * only what the routing selects (adnankhan.ai note, "Raw Abstract / Excerpt";
 * seventnews, "HGA的不同之处").  With this tier the detached history's K/V live in
 * pinned host memory, the summary tables stay in HBM (routing reads only them),
 * and after hga_route this call copies the selected history groups of every
 * (sequence, KV head) into a compact staging cache in HBM and renumbers the
 * selection for it; hga_attend_fwd / hga_attend_bwd then run on the staging cache
 * unchanged, with results bit-identical to the same calls on a cache that holds
 * the whole history in HBM.
 *
 *   k_host, v_host   [B, Hkv, host_t_cap, d] pinned host memory (hipHostMalloc, or
 *                    a pinned torch tensor) holding the history at [0, t_hist); read
 *                    by the GPU over the host link (HGA_ERR_UNSUPPORTED if not pinned)
 *   group_idx        [B, Hkv, seg_len/64, k_g] int32, as hga_route wrote it       read
 *   k_stage, v_stage [B, Hkv, stage_cap, d] device memory.  Written: rows [0, stage_hist):
 *                    slot s = the s-th distinct history group that any block of the
 *                    (sequence, KV head) selected (ascending ids), tokens 8s .. 8s+7;
 *                    rows of unused slots are not touched.  The caller places the
 *                    active segment's K/V at [stage_hist, stage_hist + seg_len).
 *   group_idx_stage  [B, Hkv, seg_len/64, k_g] int32 written: history id x -> its slot,
 *                    active id x -> stage_hist/8 + (x - t_hist/8), -1 -> -1; still
 *                    ascending.  Pass it, stage_cap as t_cap and stage_hist as t_hist
 *                    to hga_attend_fwd / hga_attend_bwd.
 *   stage_hist       a multiple of 64 of at least hga_stage_history_min() (enough for
 *                    every possible selection); stage_hist + seg_len <= stage_cap
 *                    (HGA_ERR_CAPACITY otherwise).
 * With k_g == 0 nothing is selected and the call does nothing.
 */
int hga_stage_history(const hga_shape* shape, const void* k_host, const void* v_host, int64_t host_t_cap,
                      int64_t t_hist, int64_t seg_len, const int32_t* group_idx, void* k_stage,
                      void* v_stage, int64_t stage_cap, int64_t stage_hist, int32_t* group_idx_stage,
                      void* stream);
/* Smallest valid stage_hist for hga_stage_history: min(t_hist, 8 * seg_len/64 * k_g)
 * rounded up to a multiple of 64 (-1 on a bad shape). */
int64_t hga_stage_history_min(const hga_shape* shape, int64_t t_hist, int64_t seg_len);

/* Bytes of device workspace hga_attend_bwd needs (16-byte aligned); 0 on bad shape. */
/* The workspace's first HGA_BWD_WORKSPACE_CLEAR_BYTES bytes hold counters that must
 * be zero before the workspace's first use; every call that returns HGA_OK leaves
 * them zero again, so one workspace serves any number of calls, of any shapes, with
 * no clearing in between. */
#define HGA_BWD_WORKSPACE_CLEAR_BYTES 256
size_t hga_attend_bwd_workspace_size(const hga_shape* shape, int64_t t_hist, int64_t seg_len);

/*
 * hga_attend_bwd -- gradients of hga_attend_fwd for the active segment only.
 * History tokens (< t_hist) are detached and receive nothing, and no gradient
 * flows into the summaries or the selection (adnankhan.ai note, "Raw Abstract /
 * Excerpt": only the active segment stays differentiable; seventnews,
 * "HGA的不同之处": the router has no weights of its own).
 *
 *   q, k_cache, v_cache, group_idx: as passed to hga_attend_fwd
 *   o, lse     outputs of hga_attend_fwd for the same inputs
 *   d_o        [B, Hq, seg_len, d]          upstream gradient of o
 *   dq         [B, Hq, seg_len, d]          written
 *   dk_active, dv_active [B, Hkv, seg_len, d]  written: gradients of the active
 *              keys/values k_cache[:, :, t_hist + i] (summed over every query
 *              row that attends them, across blocks and query heads)
 *   workspace  device scratch of at least hga_attend_bwd_workspace_size() bytes, at
 *              least 16-byte aligned, whose first HGA_BWD_WORKSPACE_CLEAR_BYTES bytes
 *              are zero (see above).  After HGA_ERR_HIP (a launch rejected once
 *              earlier kernels of the call were enqueued) clear them again.  Calls
 *              that share a workspace must not run concurrently.
 * The result is deterministic (no floating-point atomics; the work items' order
 * among the dK/dV work-groups varies, but each writes only its own output).
 */
int hga_attend_bwd(const hga_shape* shape, const void* q, const void* k_cache,
                   const void* v_cache, const void* o, const float* lse, const void* d_o,
                   int64_t t_cap, int64_t t_hist, int64_t seg_len, const int32_t* group_idx,
                   void* dq, void* dk_active, void* dv_active, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * hga_attend_bwd_timed -- hga_attend_bwd, plus per-kernel timing marks: for
 * kernel i of the backward (HGA_BWD_KERNELS of them, in launch order: 0 dQ,
 * rowsum(dO*O), the selection inverse and the dK/dV work list, 1 dK/dV, 2 dK/dV
 * partial sums) events[2i] is recorded on `stream` just before its launch and
 * events[2i+1] just after; a kernel that a dtype's path does not launch (the fp32
 * path has no partial sums) gets its two marks back to back.  events:
 * 2*HGA_BWD_KERNELS hipEvent_t handles created by the caller (NULL entries are
 * skipped).  Everything else as hga_attend_bwd.
 */
#define HGA_BWD_KERNELS 3
int hga_attend_bwd_timed(const hga_shape* shape, const void* q, const void* k_cache,
                         const void* v_cache, const void* o, const float* lse, const void* d_o,
                         int64_t t_cap, int64_t t_hist, int64_t seg_len, const int32_t* group_idx,
                         void* dq, void* dk_active, void* dv_active, void* workspace,
                         size_t workspace_bytes, void* const* events, void* stream);

/*
 * Generation: one new token per sequence per call.  The pages say HGA can be
 * used for generation and that a serving implementation is in development
 * (adnankhan.ai note, "Raw Abstract / Excerpt"; seventnews, "检索：密集基线无退化"),
 * without a design.  This library treats the new token at position pos[b] of
 * sequence b as a query block of one position:
 *   rows       = its Hq/Hkv query heads of KV head g
 *   candidates = chunks 0 .. J-1, J = pos[b] / 64 (every complete earlier chunk)
 *   selection  = as hga_route (max over the rows, top-k_c chunks, their groups,
 *                top-k_g groups, ties to the lower id, ascending, -1 padded)
 *   keys       = the selected groups' tokens plus its own chunk up to and
 *                including itself (positions 64J .. pos[b])
 *   summaries  = when pos[b] is the last position of its chunk (pos % 64 == 63),
 *                that chunk's group and chunk summaries are written exactly as
 *                hga_build_summaries would, so the next tokens can select it
 * Per-token routing depends on nothing after the token (strictly causal).
 *
 *   q          [B, Hq, d]               the new tokens' queries
 *   pos        [B] int32, DEVICE memory  position of each sequence's new token; its
 *              K/V must already be in the cache there.  An entry outside
 *              [0, t_cap) marks an idle slot: its chunk_idx/group_idx rows are -1,
 *              its o rows 0 and its lse -inf.
 *   chunk_sum, group_sum, k_cache, v_cache: as for the segment calls (t_cap);
 *              routing reads summary rows of chunks < J only.
 *   chunk_idx  [B, Hkv, k_c], group_idx [B, Hkv, k_g] int32
 *   o          [B, Hq, d], lse [B, Hq] float32
 *   workspace  device memory of at least hga_decode_workspace_size() bytes,
 *              16-byte aligned and zero-filled before its first use.  Every call
 *              leaves it ready for the next (its arrival counters return to zero),
 *              so it is reused without clearing; calls that share a workspace
 *              must not run concurrently.
 * Requires t_cap a multiple of 64 with t_cap/64 <= HGA_MAX_CHUNKS.
 */
size_t hga_decode_workspace_size(const hga_shape* shape, int64_t t_cap);

/* hga_decode_step -- routing, attention and the summary update (two launches).
 * chunk_sum / group_sum are read (rows of chunks < J) and updated (row J of a
 * completed chunk).  chunk_idx may be NULL (then not written). */
int hga_decode_step(const hga_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, void* chunk_sum, void* group_sum, int64_t t_cap,
                    const int32_t* pos, int32_t* chunk_idx, int32_t* group_idx, void* o,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* hga_decode_route -- the selection alone (chunk_score / group_score optional, as
 * in hga_route). */
int hga_decode_route(const hga_shape* shape, const void* q, const void* chunk_sum,
                     const void* group_sum, int64_t t_cap, const int32_t* pos,
                     int32_t* chunk_idx, int32_t* group_idx, float* chunk_score,
                     float* group_score, void* workspace, size_t workspace_bytes, void* stream);

/* hga_decode_attend -- the attention alone, over a given selection (group_idx as
 * hga_decode_route writes it; an entry outside [0, 8J) is skipped, so no read
 * leaves the token's history).  group_sum and chunk_sum (both or neither) receive
 * the summaries of completed chunks as in hga_decode_step. */
int hga_decode_attend(const hga_shape* shape, const void* q, const void* k_cache,
                      const void* v_cache, int64_t t_cap, const int32_t* pos,
                      const int32_t* group_idx, void* o, float* lse, void* group_sum,
                      void* chunk_sum, void* workspace, size_t workspace_bytes, void* stream);

/*
 * hga_decode_step_noalloc -- hga_decode_step without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  It allocates and frees
 * nothing: the generation step's workspace is a static device array inside the
 * library, HGA_DECODE_NOALLOC_MAX_BYTES bytes on each GPU it runs on, held until
 * the process ends.  Its device address is looked up on the first call on each
 * device (with that device current), which also clears the array's arrival
 * counters once, on that call's stream.
 *
 * Arguments, results and errors as hga_decode_step (with `stream` on the current
 * device), except:
 *  - HGA_ERR_WORKSPACE: the call needs more than the static array holds (more than
 *    HGA_DECODE_NOALLOC_MAX_UNITS sequence x KV-head units, or a workspace of
 *    hga_decode_workspace_size() plus the fixed counter area above
 *    HGA_DECODE_NOALLOC_MAX_BYTES: e.g. 64 sequences x 8 KV heads at 131,072 tokens
 *    and top-16 chunks / top-64 groups fit);
 *  - every call on one GPU shares that GPU's array: calls that overlap in time on
 *    one GPU (other streams, other threads) race and must be serialised by the
 *    caller; calls in one stream are ordered and safe.
 */
#define HGA_DECODE_NOALLOC_MAX_BYTES (32u << 20)
#define HGA_DECODE_NOALLOC_MAX_UNITS 16384
int hga_decode_step_noalloc(const hga_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, void* chunk_sum, void* group_sum, int64_t t_cap,
                            const int32_t* pos, int32_t* chunk_idx, int32_t* group_idx, void* o,
                            float* lse, void* stream);

/* Static description of a status code. */
const char* hga_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* HGA_H */
