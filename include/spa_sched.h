/*
 * spa_sched.h -- host-side scheduler that drives spa_unified_step across
 * decode steps: bucket-balanced phases and delayed verification.
 *
 * Pages: "SparseSpec-MLSys26" review (awesome-system-papers), 核心方法,
 * "Unified batch scheduler + fused attention kernel" (buckets count the
 * requests in each phase of the draft/verify cycle and a new request goes to
 * the emptiest one, so each step's query rows stay near (2k+1)/(k+1) B) and
 * "Delayed verification" (the requests that just verified sit out one step
 * while the host runs their accept/reject and pattern update, so that work
 * overlaps the GPU's next step); marsggbo.github.io "SparseSpec" blog,
 * sections 4.2-4.3 (4.3: the host's accept/reject work of a verify moves one
 * step later and overlaps the next step's GPU work).
 *
 * Each of `slots` batch slots holds one request.  A request's cycle is k
 * draft steps, a verify step and, with delayed verification, one step in
 * which it is not issued (the host processes its verify meanwhile): C = k+1
 * steps, or k+2 delayed.  Its phase at step t is (t + b) mod C, b its bucket.
 * At a draft step j (0-based) the request's context is c + j + 1 positions
 * (c: its committed length, the pending token at position c) and it reads the
 * list of its last verify; at its verify step the context is c + k + 1
 * positions (rows at c .. c + k, the pending token and the k drafted ones),
 * and the verify writes a new list of K = ceil(s L) positions per KV head.  A
 * verify accepts a of its k drafted tokens -- the leading run of independent
 * draws accepted with probability accept_prob -- and commits a + 1 tokens (c
 * grows by a + 1).  So the host needs a verify's outcome before the step that
 * issues its request next: the following step, or the one after it with
 * delayed verification.  A request whose generated tokens reach its target
 * retires after that verify and a new one takes its slot in the bucket holding
 * the fewest requests (lowest bucket on ties); its prompt is P =
 * prompt_min..prompt_max positions and its initial list (before its first
 * verify) is the caller's to write.  It joins its bucket at the bucket's
 * current phase: at draft phase j0 or the verify phase (j0 = k) its first
 * cycle drafts only k - j0 tokens, and its first verify keeps k+1 rows by
 * starting j0 positions early (the last j0 prompt tokens are checked again and
 * count as accepted), i.e. its committed length starts at c = P - j0; at the
 * skipped phase it starts a full cycle after it (j0 = 0).  Either way the first
 * step that issues it has context P + 1.  Random draws come from a seeded
 * splitmix64 counter generator.
 *
 * Memory: the caller passes spa_sched_bytes(cfg) bytes of host memory,
 * 64-byte aligned; the scheduler allocates nothing and keeps its whole state
 * and every array it returns there (pointers stay valid until the next call
 * on the same state).  Not thread-safe for one state.
 */
#ifndef SPA_SCHED_H_
#define SPA_SCHED_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t slots;                /* batch slots (concurrent requests), >= 1          */
  int32_t spec_k;               /* k, 1..64                                          */
  int32_t delayed;              /* 1: delayed verification                           */
  int32_t num_qo_heads;         /* H_q (logits offsets)                              */
  int32_t num_kv_heads;         /* H_kv (list offsets)                               */
  int32_t sparsity_num;         /* s = sparsity_num / sparsity_den, 0 < s <= 1       */
  int32_t sparsity_den;
  int32_t prompt_min, prompt_max; /* prompt of a new request, positions (> spec_k)    */
  int32_t output_min, output_max; /* tokens it generates before it retires (>= 1)    */
  int32_t max_len;              /* page-table row length; prompt_max + output_max + spec_k + 1 <= max_len */
  float accept_prob;            /* acceptance probability of each drafted token, [0, 1] */
  uint64_t seed;
} spa_sched_config;

/* One step's batch.  Arrays live in the scheduler state (valid until the
 * next call); is_verify .. logits_off are spa_unified_step's host arguments
 * for B requests, slot[r] is request r's batch slot: its page-table row
 * (spa_options.page_table_rows) and its list segment.  The requests listed in
 * new_slots entered since the previous step: the caller writes their initial
 * lists (new_count[i] positions per KV head in [0, new_len[i])) before
 * running the step. */
typedef struct {
  int64_t step;                 /* index of this step                                */
  int32_t B, rows;              /* requests issued, query rows                       */
  int32_t n_verify, n_draft, n_waiting, n_new;
  const uint8_t* is_verify;     /* [B] */
  const int32_t* seq_lens;      /* [B] */
  const int32_t* q_indptr;      /* [B+1] */
  const int32_t* idx_count;     /* [B] verify: K to write; draft: entries of its list */
  const int64_t* idx_off;       /* [B] element offset of the slot's list segment    */
  const int64_t* logits_off;    /* [B] verify: element offset into the step's logits */
  const int32_t* slot;          /* [B] */
  const int32_t* new_slots;     /* [n_new] */
  const int32_t* new_len;       /* [n_new] */
  const int32_t* new_count;     /* [n_new] */
  int64_t logits_elems;         /* logits elements this step writes                 */
} spa_sched_step;

/* Running totals since spa_sched_init. */
typedef struct {
  int64_t steps, verifies, drafts, waits;
  int64_t drafted;    /* drafted tokens the verifies checked */
  int64_t accepted, committed, retired, rows;
} spa_sched_stats;

/* Bytes of state for cfg (0 if cfg is invalid; spa_last_error() says why). */
size_t spa_sched_bytes(const spa_sched_config* cfg);

/* Buffer sizes a driver needs: list elements over all slots
 * (slots * H_kv * ceil(s max_len)), the most logits elements and query rows
 * one step can need. */
int32_t spa_sched_capacity(const spa_sched_config* cfg, int64_t* idx_elems,
                           int64_t* logits_elems, int32_t* rows);

/* Initialises the state: every slot gets a new request, spread over the
 * buckets. */
int32_t spa_sched_init(void* state, size_t bytes, const spa_sched_config* cfg);

/* Plans the next step (the same step again until spa_sched_commit). */
int32_t spa_sched_next(void* state, spa_sched_step* out);

/* The planned step ran: its verifies draw their accepted tokens and commit
 * them, requests that reached their target retire and new ones take their
 * slots, and the step counter advances. */
int32_t spa_sched_commit(void* state);

int32_t spa_sched_stats_read(const void* state, spa_sched_stats* out);

/* Bucket sizes (requests per phase offset), [C] with C = k+1 or k+2. */
int32_t spa_sched_buckets(const void* state, int32_t* counts, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* SPA_SCHED_H_ */
