/*
 * spa.h -- C ABI of libspa: one unified draft/verify decode-attention step
 * with PillarAttn critical-token selection, for AMD Instinct MI355X (gfx950).
 *
 * The method (pages: "SparseSpec-MLSys26" review on awesome-system-papers,
 * section 核心方法 -> PillarAttn and "Unified batch scheduler + fused
 * attention kernel"; marsggbo.github.io "SparseSpec" blog, sections 4.1-4.2):
 *   - a verify request runs full causal attention for its k+1 query rows over
 *     its whole paged context and keeps the attention logits and log-sum-exp;
 *   - the exact scores exp(logit - LSE), averaged over the k draft rows and the
 *     query heads of each GQA group, pick the top-K positions per KV head;
 *   - a draft request attends only to the positions of its stored list;
 *   - both kinds share one batch over a paged KV cache with page size 1.
 *
 * Conventions shared by every entry point
 *   Ownership   The caller owns every buffer; the library allocates and frees
 *               nothing, on the device or the host, and keeps no per-call
 *               state between calls (it caches device properties and kernel
 *               occupancies only; spa_unified_step_static alone uses a
 *               library-held device array, see there).  Device pointers (d_*) are HIP device
 *               memory; host pointers (h_*) are ordinary host memory read
 *               during the call only, except the plan buffer below.
 *   Layouts     (H_q query heads, H_kv KV heads, G = H_q / H_kv, d = head_dim,
 *               element type per spa_layout.dtype: bf16 or fp32)
 *               k_pool, v_pool  [num_slots][H_kv][d]; one slot holds one token.
 *               page_table      int32 [B][page_table_stride]; entry [r][j] is the
 *                               slot of token j of request r, valid for j < L_r
 *                               and in [0, num_slots) (out-of-range slots are
 *                               clamped, never dereferenced outside the pool).
 *               q, o            [rows][H_q][d]; a verify request owns k+1
 *                               consecutive rows (row i sits at absolute position
 *                               L_r-(k+1)+i), a draft request one row.
 *               lse             fp32 [rows][H_q], natural log.
 *               logits          fp32; verify request r owns [(k+1)][H_q][L_r]
 *                               starting at element h_logits_off[r]; entries for
 *                               positions a row cannot see are -inf.
 *               idx             int32; request r owns [H_kv][K_r] token positions
 *                               (not slots) starting at element h_idx_off[r],
 *                               ascending per KV head.
 *   Semantics   Query head h reads KV head h / G.  Softmax scale sm_scale (0 means
 *               1/sqrt(d)).  A list entry outside [0, L_r) is ignored (whatever
 *               the pool holds anywhere it is not read); a row whose list holds
 *               no valid entry gets O = 0 and LSE = -inf.  Top-K orders by
 *               (averaged score descending, position ascending).
 *   Errors      Every entry point returns an spa_status and spa_last_error()
 *               describes a non-OK one.  Arguments are checked on the host
 *               before anything is enqueued, so SPA_ERR_INVALID_ARG,
 *               SPA_ERR_UNSUPPORTED and the *_TOO_SMALL codes leave the stream
 *               and the plan buffer untouched; SPA_ERR_HIP (a failed launch or
 *               runtime call) may come after earlier launches of the same call
 *               were enqueued.
 *   Streams     Work is enqueued on `stream` (a hipStream_t; NULL = default
 *               stream) and the call returns without waiting.  Faults inside a
 *               kernel surface at the caller's next synchronisation.
 *   Workspace   d_ws/ws_bytes: caller-owned device scratch of at least
 *               spa_workspace_bytes(...) bytes for the same batch and options,
 *               256-byte aligned.  Its first 256 bytes hold the attention
 *               launches' work counters: they must be zero before a workspace
 *               is used for the first time (hipMemset, torch.zeros), and every
 *               call leaves them zero again.  The rest (split-K partials,
 *               averaged scores, a device copy of the post-pass and selection
 *               work records, the selected rows' score histograms, and for
 *               rows longer than 32,768 positions their per-chunk counts and
 *               boundary-bin candidates, 16 KiB per 8192 positions) needs no
 *               initialisation.  Calls that share one workspace must be
 *               ordered on one stream.
 *   Plan buffer h_plan/plan_bytes: caller-owned pinned host memory
 *               (hipHostMalloc, or a pinned torch tensor) of at least
 *               spa_plan_bytes(...) bytes, 64-byte aligned.  A call writes its
 *               work plan there and the kernels read it in place over the host
 *               link (no copy is enqueued).  The first 256 bytes are a header
 *               that needs no initialisation: when a buffer is passed again,
 *               the call first waits until the GPU has finished reading what
 *               the earlier call wrote (the kernels store the earlier call's
 *               sequence number into the header when they no longer read the
 *               plan; after half a second without it, or when the earlier call
 *               failed after writing the buffer, the call drains that call's
 *               device instead).  So several buffers used in turn let the host
 *               run ahead of the GPU; one buffer serialises the host on the
 *               GPU.  A buffer must stay allocated while the GPU may read it
 *               and may not be passed to two calls running concurrently on
 *               different host threads.
 *   Options     opts may be NULL (all defaults); see spa_options.  The sizes
 *               spa_workspace_bytes and spa_plan_bytes return depend on the
 *               options, so pass the same options to the size query and the
 *               call.
 *   Threads     Entry points may be called from several host threads with
 *               different plan buffers and workspaces.
 *   Graphs      Calls are not capturable into HIP graphs: a call writes its
 *               work plan into host memory at call time, so a replay would
 *               read whatever a later call left there.
 *   B == 0      is a successful no-op.
 */
#ifndef SPA_H_
#define SPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPA_ABI_VERSION 2

typedef enum {
  SPA_OK = 0,
  SPA_ERR_INVALID_ARG = 1,         /* null pointer, bad size, bad offsets ...      */
  SPA_ERR_UNSUPPORTED = 2,         /* head_dim, dtype or row count not built       */
  SPA_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < spa_workspace_bytes(...)          */
  SPA_ERR_HIP = 4,                 /* a HIP runtime call or launch failed          */
  SPA_ERR_PLAN_TOO_SMALL = 5,      /* plan_bytes < spa_plan_bytes(...)             */
  SPA_ERR_KV_FULL = 6              /* spa_kvm_*: no free device block or host chunk */
} spa_status;

typedef enum { SPA_BF16 = 0, SPA_F32 = 1 } spa_dtype;

typedef struct {
  int32_t num_qo_heads;      /* H_q, a multiple of num_kv_heads                     */
  int32_t num_kv_heads;      /* H_kv                                               */
  int32_t head_dim;          /* d: 64 or 128                                       */
  float sm_scale;            /* softmax scale; 0 selects 1/sqrt(d)                 */
  int32_t dtype;             /* spa_dtype of q, k_pool, v_pool and o              */
  int64_t num_slots;         /* rows of k_pool / v_pool                            */
  int32_t page_table_stride; /* int32 elements per page_table row (>= max L_r)    */
} spa_layout;

/* Per-call options.  Zero-initialised options (or opts == NULL) are the
 * defaults.  Results do not depend on the work split beyond floating-point
 * summation order. */
typedef struct {
  /* Positions per verify work item (split-K chunk), 0 or 1..2048.  0: the
   * longest of 2048, 1536 and 1024 that gives the batch's verify requests at
   * least two items per resident attention workgroup (two workgroups per
   * compute unit, num_cus below, when (k+1) * H_q / H_kv <= 48 on bf16, else
   * one), else 512; lengthened up to 2048 while a request would need more
   * than 256 chunks. */
  int32_t verify_chunk;
  /* List entries per draft work item, 0 or 1..2048; 0: 1024. */
  int32_t draft_chunk;
  /* Compute units the automatic verify chunk plans for; 0: 256 (MI355X).
   * Only the automatic rule reads it, so sizes stay a pure function of the
   * arguments. */
  int32_t num_cus;
  /* Nonzero: spa_unified_step on a batch holding both verify and draft
   * requests runs its draft attention as a second launch on side_stream,
   * forked from `stream` after the work already queued there (fork_event) and
   * joined back before the call's last operation (join_event), so the call as
   * a whole stays ordered on `stream` while verify attention, score averaging
   * and top-K overlap the draft attention.  The streams and events (created
   * by the caller with hipEventDisableTiming) may not be shared with calls
   * in flight on other host threads.  Other entry points ignore it. */
  int32_t overlap;
  void* side_stream;  /* hipStream_t */
  void* fork_event;   /* hipEvent_t  */
  void* join_event;   /* hipEvent_t  */
  /* Optional timing events (hipEvent_t, created by the caller; NULL entries
   * are skipped), recorded on the launch stream right before and after:
   * [0],[1] the attention launch (with overlap: the verify attention launch);
   * [2],[3] the post-pass launch (split-K merges and score averaging);
   * [4],[5] the top-K selection (with rows longer than 32,768 positions:
   * its count, per-row and chunk launches together); [6],[7] the draft
   * attention launch of an overlapped unified step (on side_stream).  A launch
   * the call does not make records nothing. */
  void* timing[8];
  /* Optional host array [B]: request r reads page_table row
   * page_table_rows[r] instead of row r, so a caller that keeps one
   * page-table row per batch slot can run any subset of its slots
   * (attention calls only; NULL: row r).  page_table_row_count is the
   * number of rows of d_page_table; every entry must lie in [0, it). */
  const int32_t* page_table_rows;
  int32_t page_table_row_count;
} spa_options;

/* Library ABI version (SPA_ABI_VERSION of the build). */
int32_t spa_abi_version(void);

/* Message describing the last non-OK status returned on this host thread. */
const char* spa_last_error(void);

/* Workspace bytes needed by spa_verify_attn, spa_pillar_topk, spa_draft_attn
 * and spa_unified_step for this batch (the largest of their needs), a pure
 * function of the arguments.  h_is_verify may be NULL (all draft) and
 * h_idx_count may be NULL for verify-only batches.  Returns 0 when the
 * arguments are invalid (spa_last_error() says why). */
size_t spa_workspace_bytes(const spa_layout* layout, int32_t B, int32_t spec_k,
                           const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                           const int32_t* h_idx_count, const spa_options* opts);

/* Plan-buffer bytes needed by the same four entry points for this batch (the
 * largest of their needs), a pure function of the arguments; 0 when they are
 * invalid. */
size_t spa_plan_bytes(const spa_layout* layout, int32_t B, int32_t spec_k,
                      const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                      const int32_t* h_idx_count, const spa_options* opts);

/* Full attention of B verify requests (k+1 rows each, rows r*(k+1)...), with
 * the logits and LSE kept.  Review of SparseSpec, PillarAttn, third bullet:
 * the verify kernel dumps attention logits and log-sum-exp on the fly.
 * h_seq_lens[B]: L_r >= k+1.  h_logits_off[B]: element offsets, each segment
 * (k+1)*H_q*L_r long and non-overlapping.  d_o [B(k+1)][H_q][d], d_lse
 * [B(k+1)][H_q]. */
int32_t spa_verify_attn(const spa_layout* layout, int32_t B, int32_t spec_k,
                        const int32_t* h_seq_lens, const int32_t* d_page_table,
                        const void* d_q, const void* d_k_pool, const void* d_v_pool, void* d_o,
                        float* d_lse, float* d_logits, const int64_t* h_logits_off, void* d_ws,
                        size_t ws_bytes, void* h_plan, size_t plan_bytes,
                        const spa_options* opts, void* stream);

/* PillarAttn selection for B verify requests.  Review of SparseSpec,
 * PillarAttn, third and fourth bullets: exact scores exp(logit - LSE) are
 * averaged over rows [avg_row_begin, avg_row_begin + avg_row_count) (the k
 * draft rows are 1..k) and the G heads of each KV head, then the top
 * h_topk[r] = K_r positions per KV head are written ascending to
 * d_idx + h_idx_off[r] as [H_kv][K_r].  d_lse [B(k+1)][H_q]; logits as above.
 * Workspace and plan sizes: spa_workspace_bytes / spa_plan_bytes of a layout
 * with these head counts, with every request a verify request and
 * h_idx_count = h_topk. */
int32_t spa_pillar_topk(int32_t B, int32_t spec_k, int32_t num_qo_heads, int32_t num_kv_heads,
                        int32_t avg_row_begin, int32_t avg_row_count, const int32_t* h_seq_lens,
                        const int32_t* h_topk, const float* d_logits,
                        const int64_t* h_logits_off, const float* d_lse, int32_t* d_idx,
                        const int64_t* h_idx_off, void* d_ws, size_t ws_bytes, void* h_plan,
                        size_t plan_bytes, const spa_options* opts, void* stream);

/* Sparse attention of B draft requests (one row each) over their stored lists.
 * Review of SparseSpec, PillarAttn, first two bullets; blog section 4.1: a
 * draft step attends only to the critical tokens.  h_idx_count[r] = list
 * length n_r >= 1 per KV head, list at d_idx + h_idx_off[r] as [H_kv][n_r]. */
int32_t spa_draft_attn(const spa_layout* layout, int32_t B, const int32_t* h_seq_lens,
                       const int32_t* d_page_table, const int32_t* h_idx_count,
                       const int64_t* h_idx_off, const int32_t* d_idx, const void* d_q,
                       const void* d_k_pool, const void* d_v_pool, void* d_o, float* d_lse,
                       void* d_ws, size_t ws_bytes, void* h_plan, size_t plan_bytes,
                       const spa_options* opts, void* stream);

/* One mixed batch: verify requests (h_is_verify[r] != 0) run spa_verify_attn
 * then spa_pillar_topk semantics and overwrite their own idx segment (K_r =
 * h_idx_count[r] entries per KV head); draft requests run spa_draft_attn over
 * the segment they own.  All attention work of both kinds goes through one
 * kernel launch.  Review of SparseSpec, "Unified batch scheduler + fused
 * attention kernel": sparse and full attention share one pipeline over
 * page-size-1 paged KV and requests of both kinds mix freely.  h_q_indptr[B+1]
 * gives each request's first q row; counts must be k+1 (verify) or 1 (draft).
 * h_logits_off[r] is read for verify requests only. */
int32_t spa_unified_step(const spa_layout* layout, int32_t B, int32_t spec_k,
                         const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                         const int32_t* h_q_indptr, const int32_t* d_page_table,
                         const void* d_q, const void* d_k_pool, const void* d_v_pool,
                         const int32_t* h_idx_count, const int64_t* h_idx_off, int32_t* d_idx,
                         void* d_o, float* d_lse, float* d_logits, const int64_t* h_logits_off,
                         int32_t avg_row_begin, int32_t avg_row_count, void* d_ws,
                         size_t ws_bytes, void* h_plan, size_t plan_bytes,
                         const spa_options* opts, void* stream);

/* Bytes of the static workspace of spa_unified_step_static (32 MiB). */
#define SPA_STATIC_WORKSPACE_BYTES (32u << 20)

/* spa_unified_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and results
 * as spa_unified_step; the workspace is a library-held device array of
 * SPA_STATIC_WORKSPACE_BYTES per GPU (held until the process ends), whose
 * address is looked up once per device on the first call made with that
 * device current.  A batch whose spa_workspace_bytes(...) exceeds it is
 * rejected with SPA_ERR_UNSUPPORTED before anything is enqueued.  The call
 * allocates nothing, on the device or in pinned host memory (the caller still
 * passes the plan buffer, inputs and outputs).  Every call on a GPU shares
 * that GPU's array: calls that may overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller.  The array's work
 * counters are zero when the library loads and every call leaves them zero;
 * nothing else in it needs to start at any value. */
int32_t spa_unified_step_static(const spa_layout* layout, int32_t B, int32_t spec_k,
                                const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                                const int32_t* h_q_indptr, const int32_t* d_page_table,
                                const void* d_q, const void* d_k_pool, const void* d_v_pool,
                                const int32_t* h_idx_count, const int64_t* h_idx_off,
                                int32_t* d_idx, void* d_o, float* d_lse, float* d_logits,
                                const int64_t* h_logits_off, int32_t avg_row_begin,
                                int32_t avg_row_count, void* h_plan, size_t plan_bytes,
                                const spa_options* opts, void* stream);

/* Recallable sparse index of B draft requests.  Page "全局的稀疏一瞥"
 * (arxiv.org 2607.27735 as rendered on bittide.aicompass.dev), section 方法,
 * Figure 3 caption: a draft's per-head index keeps the sink tokens, the
 * important history positions chosen from the last verify's attention scores,
 * and the recent tokens.  For request r and KV head g it writes, ascending, the
 * set of positions j in [0, L_r) with j < n_sink, or j >= L_r - n_recent, or j
 * an entry of the stored list d_idx_in + h_in_off[r] + g*h_in_count[r] (stored
 * entries outside [0, L_r) name no position; order and duplicates in the stored
 * list do not matter), to d_idx_out + h_out_off[r] + g*h_out_count[r], then -1
 * up to h_out_count[r] entries; spa_draft_attn and spa_unified_step ignore -1.
 * h_seq_lens[B]: the draft's current length L_r (1 <= L_r <= 1048576), so the
 * recent window holds the tokens the draft itself appended since the verify.
 * h_out_count[r] must be >= max(1, min(L_r, S + R + h_in_count[r])), S =
 * min(n_sink, L_r), R = L_r - max(S, L_r - min(n_recent, L_r)).  Output lists
 * may not overlap one another or any stored list (checked on the host from the
 * addresses); d_idx_in may be NULL when every h_in_count[r] is 0.  Plan
 * buffer: at least spa_recall_plan_bytes(B) bytes (same rules as above).  One
 * launch, then a one-thread launch that releases the plan buffer; the output
 * then feeds spa_draft_attn or the draft requests of spa_unified_step with
 * h_idx_count[r] = h_out_count[r]. */
int32_t spa_recall_index(int32_t B, int32_t num_kv_heads, const int32_t* h_seq_lens,
                         int32_t n_sink, int32_t n_recent, const int32_t* h_in_count,
                         const int64_t* h_in_off, const int32_t* d_idx_in,
                         const int32_t* h_out_count, const int64_t* h_out_off, int32_t* d_idx_out,
                         void* h_plan, size_t plan_bytes, void* stream);

/* Plan-buffer bytes of spa_recall_index for B requests (0 for B < 0). */
size_t spa_recall_plan_bytes(int32_t B);

/* Quality of index lists against one query row's exact attention.  Review
 * of SparseSpec, 核心方法 / PillarAttn, the comparison with Quest: PillarAttn
 * is judged by top-10 recall and attention coverage.  The row is row `row` of
 * B requests whose logits and LSE came from spa_verify_attn with this spec_k
 * (request r: logits [(spec_k+1)][H_q][L_r] at h_logits_off[r], LSE rows
 * r*(spec_k+1) ... of d_lse [B(spec_k+1)][H_q]); with spec_k = 1 and a draft
 * query placed in row 1, row 1 sees the draft's whole context.  For query
 * head h of request r, with p_h = exp(logit - LSE) over positions [0, L_r)
 * and the list of KV head h / G at d_list + h_list_off[r] + g*h_list_count[r]
 * (entries outside [0, L_r) name no position; repeats count once):
 *   d_top      [B][H_q][top_t]: the top_t positions of largest p_h (ties to
 *              the lower position), ascending;
 *   d_coverage [B][H_q]: the sum of p_h over the list's positions;
 *   d_recall   [B][H_q]: |top_t positions on the list| / top_t.
 * 1 <= top_t <= L_r <= 1048576.  d_ws: 16-byte aligned, at least
 * spa_list_quality_workspace_bytes(B, H_q, h_seq_lens) bytes (the rows' p_h;
 * contents on entry do not matter).  Plan buffer: at least
 * spa_list_quality_plan_bytes(B) bytes.  One launch, then a one-thread launch
 * that releases the plan buffer. */
int32_t spa_list_quality(int32_t B, int32_t spec_k, int32_t num_qo_heads, int32_t num_kv_heads,
                         int32_t row, int32_t top_t, const int32_t* h_seq_lens,
                         const float* d_logits, const int64_t* h_logits_off, const float* d_lse,
                         const int32_t* h_list_count, const int64_t* h_list_off,
                         const int32_t* d_list, int32_t* d_top, float* d_coverage,
                         float* d_recall, void* d_ws, size_t ws_bytes, void* h_plan,
                         size_t plan_bytes, void* stream);

/* Workspace bytes of spa_list_quality: sum over r of H_q * (L_r rounded up to
 * a multiple of 4) * 4.  Returns 0 for B <= 0 or a NULL pointer. */
size_t spa_list_quality_workspace_bytes(int32_t B, int32_t num_qo_heads,
                                        const int32_t* h_seq_lens);

/* Plan-buffer bytes of spa_list_quality for B requests (0 for B < 0). */
size_t spa_list_quality_plan_bytes(int32_t B);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H_ */
