/*
 * spdecode.h -- C ABI of the MI355X (gfx950) sparse decode attention library.
 *
 * Query-dependent sparse decode attention over a paged KV cache, after
 * "SparseEngine: Sparse-First Inference Engine":
 *   - Quest page selection (Appendix A.3, "Quest: Query-Dependent Page
 *     Selection"): per-page elementwise min/max key summaries, a per-page upper
 *     bound of every token's logit, top-k pages per KV head, attention over the
 *     selected pages only;
 *   - H2O eviction (Appendix A.3, "H2O: Accumulated Scores and Online
 *     Eviction"): attention probabilities added to persistent per-slot scores,
 *     then physical compaction to a fixed budget made of a recent window plus
 *     the highest-scoring older slots.
 * The five operations follow the lifecycle of Section 3.1 ("Architectural
 * Foundations"): CacheManager write/update (sp_build_page_meta),
 * build_decode_selection (sp_select_pages), the attention backend consuming an
 * AttentionView (sp_sparse_decode_attn), and finish_step's score update and
 * online eviction (sp_h2o_accumulate, sp_h2o_evict_compact).
 *
 * Conventions (all calls):
 *   - Every pointer argument other than `kv` itself is DEVICE memory on the
 *     current HIP device, except where marked "host".  The descriptor `kv` is
 *     host memory; the pointers inside it are device memory.
 *   - The caller owns all memory, including workspaces sized by
 *     sp_workspace_bytes().  The library allocates nothing and keeps no state
 *     between calls (besides the thread-local error text).
 *   - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *     NULL = the default stream).  No call synchronises the host, and no call
 *     reads device values on the host, so a sequence of calls can be captured
 *     into a HIP graph.  Per-step mutable state (lengths, slot maps, scores)
 *     lives in device buffers at stable addresses, as the pages' graph-replay
 *     rule requires (Appendix B, "CUDA Graph Execution").
 *   - Argument checks run on the host before any launch.  A failed check
 *     returns a non-zero sp_status, launches nothing, and sp_last_error()
 *     describes it.  A failed launch returns SP_ERR_HIP.
 *   - Kernels never trap.  Device-side values out of range are clamped:
 *     seq_lens above the capacity max_pages_per_seq * page_size are treated as
 *     the capacity, block ids outside [0, num_blocks) make the page be skipped.
 *   - Positions are 0-based: token/slot t of a sequence lives on logical page
 *     t / page_size at offset t % page_size (the pages' 1-based block number
 *     floor((j-1)/p), Appendix A.2, "Logical Positions and Physical Blocks").
 *
 * Physical layouts ("E" = elements per 16-byte chunk: 8 for bf16, 4 for fp32;
 * D = head_dim, P = page_size, H = num_kv_heads):
 *   k_pool     [num_blocks][H][D/E][P][E]   keys, chunk-tiled: element (t, d)
 *              of a (block, head) page sits at ((d/E)*P + t)*E + d%E.  A page of
 *              one head is one contiguous P*D*elem-byte run.
 *   v_pool     [num_blocks][H][D][P]        values, dim-major: element (t, d)
 *              at d*P + t.  Also one contiguous run per (block, head).
 *   page_meta  [num_blocks][H][2][D]        row 0 = per-channel minimum, row 1
 *              = per-channel maximum of the page's valid keys, in the KV dtype
 *              (min/max of representable values is exact).
 *   block_table[batch][max_pages_per_seq]   physical block of logical page p.
 *   seq_lens   [batch]                      tokens (Quest) or occupied slots
 *              (H2O / evicted decode) per sequence; updated on the device.
 *   q          [batch][num_q_heads][D]      in the KV dtype.
 *   Query head a reads KV head a / G with G = num_q_heads / num_kv_heads
 *   (Appendix A.1, "MHA, MQA, and GQA").
 */
#ifndef SPDECODE_H_
#define SPDECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sp_status {
  SP_OK = 0,
  SP_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  SP_ERR_BAD_SHAPE = 2,    /* a size is out of range or inconsistent */
  SP_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head_dim, page_size, dtype, mode) */
  SP_ERR_MISALIGNED = 4,   /* a device pointer is not 16-byte aligned */
  SP_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than sp_workspace_bytes() */
  SP_ERR_HIP = 6           /* a HIP launch failed; sp_last_error() holds the HIP message */
} sp_status;

typedef enum sp_dtype { SP_F32 = 0, SP_BF16 = 1 } sp_dtype;

/* Operation ids for sp_workspace_bytes(). */
enum {
  SP_OP_SELECT_PAGES = 1,
  SP_OP_DECODE_ATTN = 2,
  SP_OP_H2O_EVICT = 3,
  SP_OP_SNAPKV_SCORES = 4,
  SP_OP_H2O_PREFILL = 5,
  SP_OP_OMNIKV_SELECT = 6,
  SP_OP_QUEST_STEP = 7
};

/* Paged KV cache descriptor (host struct; pointers are device memory).
 * Supported: head_dim in {64, 128}, page_size in {16, 32}, dtype in
 * {SP_F32, SP_BF16}, num_q_heads a multiple of num_kv_heads with group
 * size G = num_q_heads / num_kv_heads <= 16. */
typedef struct sp_paged_kv {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;   /* row stride of block_table; capacity = this * page_size slots */
  int32_t num_blocks;          /* physical blocks in k_pool / v_pool / page_meta */
  int32_t dtype;               /* sp_dtype of q, pools and page_meta */
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  int32_t* seq_lens;
} sp_paged_kv;

/*
 * sp_build_page_meta -- append new tokens to the paged cache and fold their
 * keys into the page summaries; or rebuild every summary from the pool.
 *
 * Source: Appendix A.3 "Quest: Query-Dependent Page Selection" (each page keeps
 * per-channel min and max keys; new keys update their page's extrema, so the
 * summaries persist beside the KV) and Section 3.1 (CacheManager write/update).
 *
 * Append mode (n_new >= 1, k_new and v_new non-NULL):
 *   k_new, v_new  [batch][n_new][num_kv_heads][head_dim], KV dtype.
 *   Token t of sequence b is written to slot s = seq_lens[b] + t of every KV
 *   head; slots at or beyond the capacity are dropped.  If page_meta is
 *   non-NULL the page s / P gets min/max folded with the new key (a page whose
 *   first slot is written starts from the new key alone).  If slot_pos is
 *   non-NULL ([batch][num_kv_heads][slot_cap] int32), slot_pos[b][h][s] =
 *   (pos_new ? pos_new[b] : seq_lens[b]) + t, i.e. the logical position.
 *   Finally seq_lens[b] += n_new (saturating at the capacity).
 * Rebuild mode (n_new == 0, k_new == v_new == NULL, page_meta non-NULL):
 *   recomputes page_meta for pages [0, ceil(seq_lens[b] / P)) of every
 *   sequence from the pool's valid slots; seq_lens is not changed.
 * Errors: SP_ERR_NULL_PTR (kv, pools, block_table, seq_lens, or the mode's
 *   required pointers), SP_ERR_BAD_SHAPE (n_new < 0, slot_cap below the
 *   capacity when slot_pos is given), SP_ERR_UNSUPPORTED, SP_ERR_MISALIGNED.
 */
sp_status sp_build_page_meta(const sp_paged_kv* kv, const void* k_new, const void* v_new,
                             int32_t n_new, void* page_meta, const int32_t* pos_new,
                             int32_t* slot_pos, int32_t slot_cap, void* stream);

/*
 * sp_select_pages -- Quest page scoring and per-KV-head top-k.
 *
 * Source: Appendix A.3 "Quest: Query-Dependent Page Selection" (a per-page
 * estimate that upper-bounds the query-key logit of every token in the page;
 * pages are ranked by it).  The estimate for query head a is
 *   U_a(p) = sum_c max(q_{a,c} * min_{p,c}, q_{a,c} * max_{p,c})
 * and KV head h ranks its pages by S_h(p) = sum_{a : a/G = h} U_a(p) (unscaled).
 *
 *   q           [batch][num_q_heads][head_dim], KV dtype.
 *   page_meta   as produced by sp_build_page_meta.
 *   top_k       >= 1 pages kept per (sequence, KV head).
 *   sel_pages   out [batch][num_kv_heads][top_k] int32: the min(top_k, N_p)
 *               pages with the largest S (ties: lower page index), in
 *               ascending page order, padded with -1; N_p = ceil(seq_lens[b]/P)
 *               and every one of the N_p pages is a candidate.
 *   page_scores optional out [batch][num_kv_heads][max_pages_per_seq] fp32:
 *               S_h(p) for p < N_p, -INFINITY above (and for pages whose
 *               block id is out of range, which are then never preferred).
 *               May be NULL; the scores then live in the workspace.
 *   workspace   >= sp_workspace_bytes(SP_OP_SELECT_PAGES, kv, top_k) bytes,
 *               always required.  Its head holds per-(sequence, KV head)
 *               arrival counters: it must be zero-filled before its first use,
 *               and every call leaves the counters at zero.  Calls that share
 *               a workspace must not run concurrently.  Above 5120 pages
 *               per sequence the top-k runs over the scores in launches of
 *               its own, and the workspace also holds each sequence's page
 *               count and, above 32768 pages, each (sequence, KV head)'s list
 *               of kept pages (rewritten by every call; the size covers it).
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE (top_k < 1), SP_ERR_UNSUPPORTED,
 *   SP_ERR_MISALIGNED, SP_ERR_WORKSPACE.
 */
sp_status sp_select_pages(const sp_paged_kv* kv, const void* q, const void* page_meta,
                          int32_t top_k, int32_t* sel_pages, float* page_scores,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Group aggregations of the page bound for sp_select_pages_ex. */
#define SP_GROUP_SUM 0   /* S_h(p) = sum over the group's query heads of U_a(p) */
#define SP_GROUP_MAX 1   /* S_h(p) = max over the group's query heads of U_a(p) */

/*
 * sp_select_pages_ex -- sp_select_pages with pages that are always chosen
 * and a choice of group aggregation.
 *
 * Source: Section 5 (the Quest baseline configuration: 16-token pages with
 * 4 sink pages, 32 recent pages and 92 selected pages; selected budgets
 * exclude the separately listed sink and recent ones) and Appendix A.3
 * "Quest" for the bound.  For every (sequence b, KV head h) with
 * N_p = ceil(seq_lens[b] / P):
 *   forced F = pages [0, min(n_sink, N_p)) and [max(0, N_p - n_recent), N_p);
 *   chosen   = F plus the (top_k - |F|) pages outside F with the largest
 *              S_h(p) (ties: lower page index); every page if top_k >= N_p.
 * top_k is the total (4 + 32 + 92 = 128 for the configuration above).
 * group_reduce: SP_GROUP_SUM ranks by the sum of the group's per-head bounds
 * (as sp_select_pages), SP_GROUP_MAX by their largest.  page_scores (if
 * given) hold the unforced S_h(p) of the chosen aggregation.  Everything
 * else (layouts, workspace, ordering of sel_pages) is as for
 * sp_select_pages, which equals this call with n_sink = n_recent = 0 and
 * SP_GROUP_SUM.
 * Both aggregations take up to 16 query heads per KV head (the group size
 * limit of every call).
 * Errors: as sp_select_pages, plus SP_ERR_BAD_SHAPE (n_sink < 0,
 *   n_recent < 0, n_sink + n_recent > top_k, unknown group_reduce).
 */
sp_status sp_select_pages_ex(const sp_paged_kv* kv, const void* q, const void* page_meta,
                             int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t group_reduce,
                             int32_t* sel_pages, float* page_scores, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * sp_append_select_pages -- one decode token appended to every sequence and
 * the pages selected, in one launch.
 *
 * Source: Section 3.1 (the cache write of the decode step precedes
 * build_decode_selection) and Appendix A.3 "Quest" (new keys update the
 * extrema of their pages, and the page holding the newest token is a
 * candidate).  The result -- pools, page_meta, slot_pos, seq_lens, sel_pages,
 * page_scores -- is that of
 *   sp_build_page_meta(kv, k_new, v_new, 1, page_meta, pos_new, slot_pos,
 *                      slot_cap, stream);
 *   sp_select_pages_ex(kv, q, page_meta, top_k, n_sink, n_recent,
 *                      group_reduce, sel_pages, page_scores, workspace,
 *                      workspace_bytes, stream);
 * bit for bit, without the second launch.
 *   k_new, v_new  [batch][num_kv_heads][head_dim], KV dtype, 16-byte aligned
 *                 (one token per sequence; a full sequence takes none).
 *   pos_new, slot_pos, slot_cap   as for sp_build_page_meta (optional).
 *   page_meta     in/out, as for sp_build_page_meta; required.
 *   everything else as for sp_select_pages_ex; the workspace is
 *   sp_workspace_bytes(SP_OP_SELECT_PAGES, kv, top_k) bytes (its per-sequence
 *   counters serve the length update; every call leaves them at zero).
 * Errors: as sp_build_page_meta and sp_select_pages_ex.
 */
sp_status sp_append_select_pages(const sp_paged_kv* kv, const void* k_new, const void* v_new,
                                 const int32_t* pos_new, int32_t* slot_pos, int32_t slot_cap,
                                 void* page_meta, const void* q, int32_t top_k, int32_t n_sink,
                                 int32_t n_recent, int32_t group_reduce, int32_t* sel_pages,
                                 float* page_scores, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * sp_quest_decode_step -- one Quest decode step of one layer: the decode
 * token appended to every sequence, the pages selected, and every query head's
 * attention over its KV head's selected pages, in one launch.
 *
 * Source: Section 3.1 (the decode step writes the cache, builds the decode
 * selection, then runs the attention backend on the Quest AttentionView) and
 * Appendix A.3 "Quest" with Appendix A.1 "Attention over Selected
 * Positions".  The results -- pools, page_meta, slot_pos, seq_lens,
 * sel_pages, page_scores, out, lse -- are those of
 *   sp_append_select_pages(kv, k_new, v_new, pos_new, slot_pos, slot_cap,
 *                          page_meta, q, top_k, n_sink, n_recent, group_reduce,
 *                          sel_pages, page_scores, ...);
 *   sp_sparse_decode_attn(kv, q, sel_pages, top_k, scale, out, lse, NULL, 0,
 *                         ...);
 * (the same selection bit for bit; out and lse to the attention's tolerance,
 * the split of the attention over workgroups being different).
 *   k_new, v_new  [batch][num_kv_heads][head_dim] or both NULL (no append:
 *                 select and attend over the cache as it is).
 *   every other argument as for those two calls; the attention is sparse
 *   (sel_pages is an output) and writes no logits.
 *   workspace     >= sp_workspace_bytes(SP_OP_QUEST_STEP, kv, top_k) bytes,
 *                 zero-filled before its first use, and used for calls of one
 *                 descriptor shape and top_k (zero-fill it again before
 *                 another).  It carries per-unit epochs from call to call;
 *                 every call leaves its arrival counters at zero.  Its error
 *                 word (the int at byte offset sp_quest_step_error_offset(kv))
 *                 stays 0; it is set to 1 only if a workgroup's wait for
 *                 another's selection or split state gave up, which cannot
 *                 happen while the launch is resident.
 * The single launch needs every workgroup resident at once,
 * max_pages_per_seq <= 12288 (6144 for fp32 caches), num_blocks < 2^25, and either the sum over the
 * group (SP_GROUP_SUM) or the maximum (SP_GROUP_MAX) with bf16 and
 * head_dim 128; otherwise the call runs the two launches above on the same
 * workspace (sp_quest_step_single_launch tells which).
 * Errors: those of the two calls, plus SP_ERR_UNSUPPORTED for num_blocks >=
 *   2^25 and SP_ERR_NULL_PTR for exactly one of k_new, v_new.
 */
sp_status sp_quest_decode_step(const sp_paged_kv* kv, const void* k_new, const void* v_new,
                               const int32_t* pos_new, int32_t* slot_pos, int32_t slot_cap,
                               void* page_meta, const void* q, int32_t top_k, int32_t n_sink,
                               int32_t n_recent, int32_t group_reduce, float scale, int32_t* sel_pages,
                               float* page_scores, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Byte offset of the fused step's error word in its workspace (host only). */
size_t sp_quest_step_error_offset(const sp_paged_kv* kv);

/*
 * sp_quest_step_single_launch -- whether sp_quest_decode_step runs as one
 * launch (*single_launch = 1) or as the two launches (0) for this descriptor
 * and group_reduce on the current device.  Host only: reads the kernel's
 * occupancy from the runtime and launches nothing.
 * Errors: SP_ERR_NULL_PTR (kv or single_launch NULL), the descriptor errors
 *   of every call, SP_ERR_BAD_SHAPE for a group_reduce other than
 *   SP_GROUP_SUM / SP_GROUP_MAX.
 */
sp_status sp_quest_step_single_launch(const sp_paged_kv* kv, int32_t group_reduce, int32_t* single_launch);

/*
 * sp_sparse_decode_attn -- decode attention of every query head over either
 * the selected pages (Quest) or all occupied slots (dense; H2O and evicted
 * decode).
 *
 * Source: Appendix A.1 "Attention over Selected Positions" (attention over a
 * nonempty selected set normalises over the selected positions; dense decode
 * uses all of them) and Appendix A.3 "Quest" (attention uses the actual KV of
 * the selected pages).  For query head a of sequence b over token set T:
 *   z_j = scale * (q_a . k_j),  out_a = sum_{j in T} softmax_T(z)_j v_j,
 *   lse_a = log sum_{j in T} exp(z_j)   (natural log).
 *
 *   q          [batch][num_q_heads][head_dim], KV dtype.
 *   sel_pages  [batch][num_kv_heads][top_k] logical pages (entries < 0 or
 *              >= ceil(seq_lens[b]/P) are ignored; entries must be distinct),
 *              or NULL for dense mode (T = slots [0, seq_lens[b])).
 *   top_k      row length of sel_pages (>= 1); ignored in dense mode.
 *   out        out [batch][num_q_heads][head_dim] fp32.  A sequence with an
 *              empty T gets out = 0 and lse = -INFINITY.
 *   lse        optional out [batch][num_q_heads] fp32.
 *   logits     optional out [batch][num_q_heads][logit_cap] fp32, dense mode
 *              only: z_j for j < seq_lens[b] (other entries untouched).
 *              logit_cap >= max_pages_per_seq * page_size.
 *   workspace  >= sp_workspace_bytes(SP_OP_DECODE_ATTN, kv, top_k) bytes:
 *              per-(sequence, KV head) arrival counters, then the split
 *              softmax states (and, in dense mode with more than 2048
 *              sequences, the per-sequence tile prefix, written by a launch
 *              of its own before the attention).  It must be zero-filled
 *              before its first use; every call leaves the counters at zero.
 *              Calls that share a workspace must not run concurrently.
 * Limits: a call streams fewer than 2^31 16-token tiles; otherwise
 *   SP_ERR_UNSUPPORTED.
 * Accumulation is fp32; bf16 inputs use MFMA for the G-head QK^T and PV tiles.
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED (logits with
 *   sel_pages), SP_ERR_MISALIGNED, SP_ERR_WORKSPACE.
 */
sp_status sp_sparse_decode_attn(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages,
                                int32_t top_k, float scale, float* out, float* lse,
                                float* logits, int32_t logit_cap, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * sp_sparse_decode_attn_noalloc -- sp_sparse_decode_attn without a caller
 * workspace, for callers that cannot allocate device memory: code running
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, modes, kernels and results (bit for bit) as
 * sp_sparse_decode_attn, minus workspace / workspace_bytes.
 *
 * The arrival counters and split records live in a scratch array inside the
 * library, one per GPU: SP_NOALLOC_SCRATCH_BYTES bytes of device memory that
 * the library holds on every device it runs on until the process ends (the
 * first SP_NOALLOC_COUNTER_BYTES hold the counters, the rest the records).
 * The first call on a device looks the array up and clears its counters with
 * a fill kernel on `stream`; every call leaves them at zero.  The call
 * allocates nothing.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, threads or processes' graphs replayed concurrently) race
 * and give wrong results.  Order them on one stream.
 * Limits: batch * num_kv_heads <= SP_NOALLOC_COUNTER_BYTES / 4, and the call's
 *   split records, (workgroups + batch * num_kv_heads) * G * (head_dim + 2) * 4
 *   bytes with at most 1024 workgroups, within the remaining
 *   SP_NOALLOC_SCRATCH_BYTES - SP_NOALLOC_COUNTER_BYTES bytes (batch 256 with 8
 *   KV heads, G = 4 and head_dim 128 needs 5.3 MB).  Larger shapes return
 *   SP_ERR_UNSUPPORTED; they need sp_sparse_decode_attn with a workspace.
 * Errors: those of sp_sparse_decode_attn except SP_ERR_WORKSPACE, plus
 *   SP_ERR_HIP if the scratch array cannot be looked up on this device.
 */
#define SP_NOALLOC_SCRATCH_BYTES (16u << 20)
#define SP_NOALLOC_COUNTER_BYTES (64u << 10)
sp_status sp_sparse_decode_attn_noalloc(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages,
                                        int32_t top_k, float scale, float* out, float* lse,
                                        float* logits, int32_t logit_cap, void* stream);

/*
 * sp_h2o_accumulate -- add this step's attention probabilities to the
 * persistent per-slot scores.
 *
 * Source: Appendix A.3 "H2O: Accumulated Scores and Online Eviction"
 * (attention over the available set adds its weights to persistent scores; the
 * newest token starts from zero before this update).  Under GQA the score of a
 * KV-head slot is the sum over the group's query heads:
 *   for j < L_b = seq_lens[b]:
 *     s[b][h][j] = (j >= L_b - n_new ? 0 : s[b][h][j])
 *                  + sum_{a : a/G = h} exp(logits[b][a][j] - lse[b][a]).
 *
 *   logits, lse  as written by sp_sparse_decode_attn in dense mode.
 *   n_new        slots appended this step (>= 0) whose old score is reset.
 *   scores       in/out [batch][num_kv_heads][slot_cap] fp32.
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE (n_new < 0, logit_cap or slot_cap
 *   below the capacity), SP_ERR_MISALIGNED.
 */
sp_status sp_h2o_accumulate(const sp_paged_kv* kv, const float* logits, const float* lse,
                            int32_t logit_cap, int32_t n_new, float* scores, int32_t slot_cap,
                            void* stream);

/*
 * sp_decode_attn_accumulate -- dense decode attention over the occupied slots
 * with the H2O score update of the same step fused in: the result of
 * sp_sparse_decode_attn(kv, q, NULL, 0, scale, out, lse, logits, logit_cap,
 * ...) followed by sp_h2o_accumulate(kv, logits, lse, logit_cap, n_new,
 * scores, slot_cap), bit for bit, in one launch.
 *
 * Source: Appendix A.1 "Attention over Selected Positions" (dense decode over
 * the full available set) and Appendix A.3 "H2O: Accumulated Scores and
 * Online Eviction" (the step's attention weights are added to the persistent
 * scores; the newest token starts from zero).  The workgroup that finishes a
 * (sequence, KV head) -- the one that writes its lse -- updates that unit's
 * scores from the logits.
 *
 *   q, scale, out, lse, logits, logit_cap, workspace
 *              as sp_sparse_decode_attn in dense mode (lse and logits are
 *              required here; workspace sized by
 *              sp_workspace_bytes(SP_OP_DECODE_ATTN, kv, 0)).
 *   n_new, scores, slot_cap
 *              as sp_h2o_accumulate.
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED,
 *   SP_ERR_MISALIGNED, SP_ERR_WORKSPACE, as the two calls it replaces.
 */
sp_status sp_decode_attn_accumulate(const sp_paged_kv* kv, const void* q, float scale, float* out,
                                    float* lse, float* logits, int32_t logit_cap, int32_t n_new,
                                    float* scores, int32_t slot_cap, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * sp_h2o_evict_compact -- H2O online eviction with physical, order-preserving
 * compaction of the retained slots.
 *
 * Source: Appendix A.3 "H2O" (retained set = a protected recent window of at
 * most B positions plus the highest-scoring other tokens; KV outside it is
 * evicted and retained scores persist) and Section 3.1 (physical eviction
 * updates retained-slot mappings and context lengths).
 * Precondition: for every (b, h) the occupied slots [0, seq_lens[b]) hold
 * strictly increasing logical positions (true when appends use increasing
 * positions and only this call removes slots), so the recent window is the
 * last recent_window slots and "lower slot" means "lower position".
 * For every sequence with L = seq_lens[b] > budget and every KV head:
 *   keep slots [L - recent_window, L) and the (budget - recent_window) slots of
 *   [0, L - recent_window) with the largest scores (ties: lower slot); move the
 *   kept slots' K, V, score and slot_pos (if non-NULL) down to slots
 *   [0, budget) in their original order; then seq_lens[b] = budget.
 * Sequences with seq_lens[b] <= budget are untouched.
 *
 *   scores     in/out [batch][num_kv_heads][slot_cap] fp32.
 *   slot_pos   optional in/out [batch][num_kv_heads][slot_cap] int32.
 *   workspace  sp_workspace_bytes(SP_OP_H2O_EVICT, kv, budget) bytes, 16-byte
 *              aligned.  Above a capacity of 8192 slots it is required and
 *              holds a per-(sequence, KV head) list of the kept slots (no state
 *              between calls).  Up to 8192 slots it is optional and holds one
 *              counter per sequence, through which the last KV head to finish
 *              sets the length inside the eviction kernel; the counters must
 *              be zero before first use (every call leaves them zero), and
 *              calls sharing it must not overlap.  With NULL or a smaller
 *              buffer the length update is a second launch; results are the
 *              same either way.
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE (budget < 1, recent_window < 0 or
 *   > budget, slot_cap below the capacity), SP_ERR_UNSUPPORTED, SP_ERR_MISALIGNED,
 *   SP_ERR_WORKSPACE.
 */
sp_status sp_h2o_evict_compact(const sp_paged_kv* kv, float* scores, int32_t* slot_pos,
                               int32_t slot_cap, int32_t budget, int32_t recent_window,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * sp_snapkv_scores -- SnapKV selection scores of the prompt positions from an
 * observation window.
 *
 * Source: Appendix A.3 "SnapKV: Prompt Selection from an Observation Window"
 * (the last w prompt positions are the observation window; each earlier
 * position accumulates the attention the window's queries give it; a
 * one-dimensional max pooling of width kappa gives the selection score) and
 * Section 5 (a window of 32 and a pooling kernel of 7 in the compared setup).
 * The prompt is slots [0, L), L = seq_lens[b], holding positions 0 .. L-1 in
 * order; window query i (0 <= i < w = n_obs) sits at position L - w + i.
 * For every sequence with L > w, every KV head h and j < L - w:
 *   u(j) = sum_{i < w} sum_{a : a/G = h} softmax_{t <= L-w+i}(scale * q[b][i][a] . k_t)[j]
 *   scores[b][h][j] = +inf                                  if j < n_sink,
 *                     max { u(r) : |r - j| <= pool_kernel/2, 0 <= r < L - w }  otherwise.
 * Slots j >= L - w are not written (the window is always retained); nothing
 * is written for sequences with L <= w.  Followed by
 * sp_h2o_evict_compact(kv, scores, ..., budget, recent_window = n_obs) this
 * keeps the window, the sinks and the best-pooled earlier positions (ties:
 * lower position) and compacts them physically.
 *
 *   q_obs       device [batch][n_obs][num_q_heads][head_dim] bf16, 16-byte
 *               aligned: the window queries (after any positional rotation).
 *   n_obs       w >= 1; num_q_heads / num_kv_heads * n_obs <= 4096.
 *   scale       softmax temperature, finite and > 0 (usually 1/sqrt(head_dim)).
 *   pool_kernel kappa in [1, 257]; the window is [j - kappa/2, j + kappa/2]
 *               (integer division), clipped to the earlier positions.
 *   n_sink      >= 0: earlier positions j < n_sink score +inf.
 *   scores      device out [batch][num_kv_heads][slot_cap] fp32.
 *   workspace   >= sp_workspace_bytes(SP_OP_SNAPKV_SCORES, kv, n_obs) bytes,
 *               16-byte aligned; no state is kept in it between calls.
 * Block-table entries of the pages holding slots [0, L) must be valid block
 * ids (others read block 0; the result is then unspecified).  bf16 caches
 * only.  Products are fp32 (v_mfma_f32_16x16x32_bf16), softmax in fp32.
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED (fp32 cache, or
 *   batch * num_kv_heads > 65535), SP_ERR_MISALIGNED, SP_ERR_WORKSPACE.
 */
sp_status sp_snapkv_scores(const sp_paged_kv* kv, const void* q_obs, int32_t n_obs, float scale,
                           int32_t pool_kernel, int32_t n_sink, float* scores, int32_t slot_cap,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * sp_h2o_prefill_scores -- H2O score accumulation for one prefill chunk.
 *
 * Source: Appendix A.3 "H2O: Accumulated Scores and Online Eviction" (attention
 * over the available set adds its weights to persistent scores; a new token
 * starts from zero) with the chunk-wise prefill eviction of Section 3.1
 * ("Fine-Grained Lifecycle Hooks": finish_step evicts per prefill chunk) and
 * the FP32 probability scoring of Appendix C.1.
 * Precondition: the chunk's n_q tokens were just appended, so for every
 * sequence with L = seq_lens[b] >= n_q the chunk is slots [L - n_q, L) and
 * slots [0, L - n_q) hold the retained earlier entries (positions below the
 * chunk's, in ascending order).  Chunk query i sees slots [0, L - n_q + i].
 * For every such sequence, KV head h and slot j < L:
 *   scores[b][h][j] = (j >= L - n_q ? 0 : scores[b][h][j])
 *     + sum_{i < n_q} sum_{a : a/G = h} softmax_{t <= L-n_q+i}(scale * q[b][i][a] . k_t)[j].
 * Sequences with L < n_q are untouched.  Follow with sp_h2o_evict_compact to
 * evict down to the budget after the chunk.
 *
 *   q_chunk     device [batch][n_q][num_q_heads][head_dim] bf16, 16-byte
 *               aligned: the chunk's queries (after positional rotation).
 *   n_q         1 <= n_q <= 65536.
 *   scale       finite and > 0.
 *   scores      device in/out [batch][num_kv_heads][slot_cap] fp32.
 *   workspace   >= sp_workspace_bytes(SP_OP_H2O_PREFILL, kv, n_q) bytes,
 *               16-byte aligned; no state is kept in it between calls.
 * The rows (query, query head) are processed in passes of as many 256-row
 * slabs as keep the per-slab column sums (batch * num_kv_heads * capacity
 * floats each) within 256 MiB, and at least 16; the workspace grows with n_q
 * up to that pass size.  The sums are deterministic.  bf16 caches only.
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED (fp32 cache, or
 *   batch * num_kv_heads > 65535), SP_ERR_MISALIGNED, SP_ERR_WORKSPACE.
 */
sp_status sp_h2o_prefill_scores(const sp_paged_kv* kv, const void* q_chunk, int32_t n_q, float scale,
                                float* scores, int32_t slot_cap, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * sp_omnikv_select -- OmniKV token selection at an observation layer.
 *
 * Source: Appendix A.3 "OmniKV" (an observation layer ranks every position by
 * its largest query-key logit across heads and keeps a selected-token budget
 * b; the sparse layers assigned to it reuse those positions over their own
 * caches) and Section 3.1 ("Fine-Grained Lifecycle Hooks": on_layer_end with
 * build_decode_selection passes the indices between layers).
 * For every sequence with L = seq_lens[b] and every slot j < L:
 *   token_scores[b][j] = max_{a < num_q_heads} q[b][a] . k_{a / G}[j]   (unscaled)
 * The selection is the top_b slots by that score (ties: lower slot), or every
 * slot when L <= top_b, the same for all KV heads.  It is written as page
 * entries of the sparse-attention selection format, ascending:
 *   sel_pages[b][h][e] = page p, sel_mask[b][h][e] = bit t set for slot p*P + t
 * selected; entries past the last selected page are -1 with mask 0.
 *
 *   q             device [batch][num_q_heads][head_dim] bf16, 16-byte aligned:
 *                 the observation layer's current queries.
 *   top_b         >= 1.
 *   sel_pages     device out [batch][num_kv_heads][k_pages] int32.
 *   sel_mask      device out [batch][num_kv_heads][k_pages] uint32 (P <= 32).
 *   k_pages       >= min(top_b, max_pages_per_seq): room for any selection.
 *   token_scores  device out [batch][slot_cap] fp32 (also the ranking buffer).
 *   workspace     >= sp_workspace_bytes(SP_OP_OMNIKV_SELECT, kv, top_b) bytes,
 *                 16-byte aligned; no state between calls.
 * bf16 caches, num_q_heads <= 128, at most 16 query heads per KV head.  The
 * logits are fp32 sums of exact bf16 products (v_mfma_f32_16x16x32_bf16).
 * A sparse layer then calls
 * sp_sparse_decode_attn_masked(kv_of_that_layer, q_of_that_layer, sel_pages,
 * sel_mask, k_pages, ...).
 * Errors: SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED,
 *   SP_ERR_MISALIGNED, SP_ERR_WORKSPACE.
 */
sp_status sp_omnikv_select(const sp_paged_kv* kv, const void* q, int32_t top_b, int32_t* sel_pages,
                           uint32_t* sel_mask, int32_t k_pages, float* token_scores, int32_t slot_cap,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * sp_sparse_decode_attn_masked -- sparse decode attention over selected pages,
 * restricted to the selected tokens of each page.
 *
 * Source: Appendix A.1 "Attention over Selected Positions" (softmax over the
 * selected positions only); the selection is token-granular, as OmniKV's
 * reused positions, and carried as pages plus token masks.
 * As sp_sparse_decode_attn in sparse mode (out, lse, workspace the same; no
 * logits), except that slot p*P + t of entry (p, mask) is attended only when
 * bit t of the mask is set (and the slot is below seq_lens[b]).  Every head
 * must have at least one attended slot (else out = 0, lse = -inf).
 * Errors: as sp_sparse_decode_attn.
 */
sp_status sp_sparse_decode_attn_masked(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages,
                                       const uint32_t* sel_mask, int32_t top_k, float scale, float* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Workspace bytes an operation needs for this descriptor (host only; never
 * touches the device).  For SP_OP_DECODE_ATTN pass the call's top_k, or 0 for
 * dense mode; for SP_OP_H2O_EVICT the budget (0: enough for any budget); for
 * SP_OP_SNAPKV_SCORES n_obs; for SP_OP_H2O_PREFILL n_q; for
 * SP_OP_OMNIKV_SELECT top_b.  Returns 0 for an unknown op or an invalid
 * descriptor. */
size_t sp_workspace_bytes(int32_t op, const sp_paged_kv* kv, int32_t top_k);

/* Static name of a status code (host only): status is an sp_status value;
 * any other value gives "SP_ERR_UNKNOWN".  Taken as int32_t so that any value
 * may be passed. */
const char* sp_status_str(int32_t status);

/* Thread-local text describing the last non-OK return on this thread (host
 * only; empty string if none).  Valid until the next call on this thread. */
const char* sp_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch (host only). */
int32_t sp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPDECODE_H_ */
