/*
 * oracle.c -- plain, slow, fp64 reference of one unified draft/verify
 * decode-attention step with PillarAttn top-K selection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header,
 * table or helper with the HIP library; the only thing both sides consume is
 * the seeded input batch.
 *
 * What each function follows (pages: "SparseSpec-MLSys26" on
 * awesome-system-papers.pages.dev, the review; marsggbo.github.io "SparseSpec"
 * blog):
 *   oracle_verify_request  full causal attention of the k+1 verify query rows,
 *                          with logits and log-sum-exp kept (review, 核心方法 /
 *                          PillarAttn, third bullet; blog section 4.1).
 *   oracle_average         exact scores exp(logit - LSE), averaged over the k
 *                          draft rows and the query heads of one GQA group
 *                          (review, PillarAttn, third and fourth bullets).
 *   oracle_topk            top-K of the averaged scores per KV head (review,
 *                          PillarAttn, first and fourth bullets; s = 0.05).
 *   oracle_draft_request   attention of one draft row restricted to its index
 *                          list (review, PillarAttn, second bullet; blog 4.1).
 *   oracle_step            the whole unified batch: verify requests run the
 *                          first three, draft requests the last (review,
 *                          "Unified batch scheduler + fused attention kernel").
 *   oracle_list_quality    how well an index list covers one query row's exact
 *                          attention: attention coverage (softmax mass on the
 *                          list) and recall of the row's exact top-T (review,
 *                          核心方法 / PillarAttn, the comparison with Quest:
 *                          top-10 recall and attention coverage).
 *   oracle_recall_index    the recallable per-head index of a draft step: sink
 *                          tokens, the stored important positions and the
 *                          recent tokens (arxiv.org 2607.27735 as rendered on
 *                          bittide.aicompass.dev, "全局的稀疏一瞥", section 方法,
 *                          Figure 3 caption).
 *
 * Readings where the pages are silent (each is exercised by a test):
 *   - softmax scale is a parameter (callers use 1/sqrt(d));
 *   - verify row i of a request with L tokens sits at absolute position
 *     L-(k+1)+i and sees positions j <= L-(k+1)+i (standard causal decoding);
 *     hidden positions get logit -inf;
 *   - query head h belongs to KV head h / (H_q/H_kv);
 *   - the averaged rows are [row_begin, row_begin+row_count) (default 1..k, the
 *     rows carrying the k draft tokens); the mean is over (row, head) pairs;
 *   - top-K orders by (score descending, position ascending) and returns the
 *     chosen positions ascending;
 *   - a draft list entry outside [0, L) is ignored; if none remains, O = 0 and
 *     LSE = -inf; duplicate entries are attended as many times as listed;
 *   - the recallable index is a set: sinks are positions [0, n_sink), recent
 *     tokens are the last n_recent positions [L - n_recent, L) of the draft's
 *     current length L (so they include the tokens the draft itself appended),
 *     and each position appears once; the pages give neither count.
 *
 * Arithmetic is fp64; bf16 inputs are widened exactly.
 *
 * Mutants: building with -DORACLE_MUTANT=n plants one deliberate mistake (see
 * the MUT() uses below); the test suite uses them to show that its pins catch
 * each kind of slip.  A normal build has ORACLE_MUTANT == 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(n) (ORACLE_MUTANT == (n))

/* ---- element access ---------------------------------------------------- */
/* dtype 0: bf16 stored as its 16 high bits of an IEEE binary32; dtype 1: fp32 */
static double load_elem(const void* base, int64_t i, int dtype) {
  if (dtype == 0) {
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/* K or V row of KV head g stored at pool slot `slot`: [slots][Hkv][d] */
static int64_t kv_index(int64_t slot, int g, int c, int Hkv, int d) {
  if (MUT(12)) return (slot * d + c) * (int64_t)Hkv + g; /* layout read as [slots][d][Hkv] */
  return (slot * Hkv + g) * (int64_t)d + c;
}

static int kv_head_of(int h, int Hq, int Hkv) {
  int G = Hq / Hkv;
  if (MUT(3)) return h % Hkv;
  return h / G;
}

/* ---- full attention of the verify rows ----------------------------------
 * q       [(k+1)][Hq][d]       the k+1 query rows of the request
 * pt_row  [L]                  token position -> pool slot
 * logits  [(k+1)][Hq][L]       out: sm_scale * <q, K>, -inf where hidden
 * lse     [(k+1)][Hq]          out: natural-log log-sum-exp over visible j
 * o       [(k+1)][Hq][d]       out: softmax-weighted sum of V rows
 */
void oracle_verify_request(int Hq, int Hkv, int d, double sm_scale, int dtype, int L, int k,
                           const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* pt_row, double* logits, double* lse, double* o) {
  const int rows = k + 1;
  const double scale = MUT(4) ? 1.0 : sm_scale;
  for (int i = 0; i < rows; ++i) {
    int last_visible = L - (k + 1) + i;           /* absolute position of row i */
    if (MUT(1)) last_visible = L - 1;
    if (MUT(2)) last_visible = L - (k + 1) + i - 1;
    for (int h = 0; h < Hq; ++h) {
      const int g = kv_head_of(h, Hq, Hkv);
      double* lrow = logits + ((int64_t)i * Hq + h) * L;
      for (int j = 0; j < L; ++j) {
        if (j > last_visible) {
          lrow[j] = -INFINITY;
          continue;
        }
        const int64_t slot = pt_row[j];
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
          dot += load_elem(q, ((int64_t)i * Hq + h) * d + c, dtype) *
                 load_elem(k_pool, kv_index(slot, g, c, Hkv, d), dtype);
        lrow[j] = scale * dot;
      }
      double m = -INFINITY;
      for (int j = 0; j < L; ++j)
        if (lrow[j] > m) m = lrow[j];
      double sum = 0.0;
      for (int j = 0; j < L; ++j)
        if (lrow[j] != -INFINITY) sum += exp(lrow[j] - m);
      const double this_lse = MUT(5) ? log(sum) : m + log(sum);
      lse[i * Hq + h] = this_lse;
      double* orow = o + ((int64_t)i * Hq + h) * d;
      for (int c = 0; c < d; ++c) orow[c] = 0.0;
      for (int j = 0; j < L; ++j) {
        if (lrow[j] == -INFINITY) continue;
        const double p = exp(lrow[j] - (MUT(5) ? m + log(sum) : this_lse));
        const int64_t slot = MUT(11) ? j : pt_row[j];
        for (int c = 0; c < d; ++c)
          orow[c] += p * load_elem(v_pool, kv_index(slot, g, c, Hkv, d), dtype);
      }
    }
  }
}

/* ---- score rematerialisation and averaging -------------------------------
 * pbar[g][j] = 1/(n G) * sum_{i in [a, a+n)} sum_{h in group g} exp(logit[i][h][j] - lse[i][h])
 * logits  [(k+1)][Hq][L], lse [(k+1)][Hq]; pbar out [Hkv][L].
 */
void oracle_average(int Hq, int Hkv, int L, int k, int row_begin, int row_count,
                    const double* logits, const double* lse, double* pbar) {
  const int G = Hq / Hkv;
  (void)k;
  for (int64_t x = 0; x < (int64_t)Hkv * L; ++x) pbar[x] = 0.0;
  int a = row_begin;
  if (MUT(6)) a = 0;
  for (int i = a; i < a + row_count; ++i) {
    for (int h = 0; h < Hq; ++h) {
      const int g = kv_head_of(h, Hq, Hkv);
      const double* lrow = logits + ((int64_t)i * Hq + h) * L;
      const double l = lse[i * Hq + h];
      for (int j = 0; j < L; ++j) {
        if (lrow[j] == -INFINITY) continue;
        pbar[(int64_t)g * L + j] += exp(lrow[j] - l);
      }
    }
  }
  const double norm = MUT(7) ? (double)row_count : (double)row_count * G;
  for (int64_t x = 0; x < (int64_t)Hkv * L; ++x) pbar[x] /= norm;
}

/* ---- top-K ---------------------------------------------------------------
 * Brute force: order every position by (score descending, position
 * ascending), keep the first K, and return them ascending.
 */
typedef struct {
  double s;
  int32_t j;
} scored_pos;

static int by_score_then_pos(const void* pa, const void* pb) {
  const scored_pos* a = (const scored_pos*)pa;
  const scored_pos* b = (const scored_pos*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  if (MUT(8)) return (a->j > b->j) ? -1 : (a->j < b->j);
  return (a->j < b->j) ? -1 : (a->j > b->j);
}

static int by_pos(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a < b) ? -1 : (a > b);
}

int oracle_topk(int L, int K, const double* score, int32_t* idx_out) {
  if (K < 1 || K > L) return -1;
  scored_pos* all = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)L);
  if (!all) return -2;
  for (int j = 0; j < L; ++j) {
    all[j].s = score[j];
    all[j].j = j;
  }
  qsort(all, (size_t)L, sizeof(scored_pos), by_score_then_pos);
  for (int t = 0; t < K; ++t) idx_out[t] = all[t].j;
  free(all);
  if (!MUT(9)) qsort(idx_out, (size_t)K, sizeof(int32_t), by_pos);
  return 0;
}

/* ---- sparse attention of one draft row -----------------------------------
 * q    [Hq][d]; idx [Hkv][n_idx] token positions; o out [Hq][d]; lse out [Hq].
 */
void oracle_draft_request(int Hq, int Hkv, int d, double sm_scale, int dtype, int L,
                          const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* pt_row, int n_idx, const int32_t* idx,
                          double* o, double* lse) {
  double* lg = (double*)malloc(sizeof(double) * (size_t)(n_idx > 0 ? n_idx : 1));
  for (int h = 0; h < Hq; ++h) {
    const int g = kv_head_of(h, Hq, Hkv);
    const int32_t* list = idx + (int64_t)g * n_idx;
    double m = -INFINITY;
    for (int t = 0; t < n_idx; ++t) {
      int32_t pos = list[t];
      if (!MUT(10) && (pos < 0 || pos >= L)) {
        lg[t] = -INFINITY;
        continue;
      }
      if (MUT(10)) pos = pos < 0 ? 0 : (pos >= L ? L - 1 : pos);
      const int64_t slot = pt_row[pos];
      double dot = 0.0;
      for (int c = 0; c < d; ++c)
        dot += load_elem(q, (int64_t)h * d + c, dtype) *
               load_elem(k_pool, kv_index(slot, g, c, Hkv, d), dtype);
      lg[t] = sm_scale * dot;
      if (lg[t] > m) m = lg[t];
    }
    double* orow = o + (int64_t)h * d;
    for (int c = 0; c < d; ++c) orow[c] = 0.0;
    if (m == -INFINITY) {
      lse[h] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int t = 0; t < n_idx; ++t)
      if (lg[t] != -INFINITY) sum += exp(lg[t] - m);
    lse[h] = m + log(sum);
    for (int t = 0; t < n_idx; ++t) {
      if (lg[t] == -INFINITY) continue;
      const double p = exp(lg[t] - lse[h]);
      int32_t pos = list[t];
      if (MUT(10)) pos = pos < 0 ? 0 : (pos >= L ? L - 1 : pos);
      const int64_t slot = pt_row[pos];
      for (int c = 0; c < d; ++c)
        orow[c] += p * load_elem(v_pool, kv_index(slot, g, c, Hkv, d), dtype);
    }
  }
  free(lg);
}

/* ---- one unified step over a batch ---------------------------------------- */
typedef struct {
  int B, k, Hq, Hkv, d, dtype, row_begin, row_count;
  double sm_scale;
  const uint8_t* is_verify;
  const int32_t* seq_lens;
  const int32_t* q_indptr;
  const int32_t* page_table;
  int64_t pt_stride;
  const void *q, *k_pool, *v_pool;
  const int32_t* idx_count;
  const int64_t* idx_off;
  int32_t* idx;          /* drafts read their segment, verifies write theirs */
  double* o;             /* [rows][Hq][d] */
  double* lse;           /* [rows][Hq] */
  double* logits;        /* verify r at logits_off[r] */
  const int64_t* logits_off;
  const uint8_t* selected; /* optional: only these requests are computed */
  int next;              /* work counter */
  int status;
  pthread_mutex_t lock;
} step_args;

static int q_elem_bytes(int dtype) { return dtype == 0 ? 2 : 4; }

static int run_request(step_args* a, int r) {
  const int Hq = a->Hq, Hkv = a->Hkv, d = a->d, L = a->seq_lens[r];
  const int32_t* pt_row = a->page_table + (int64_t)r * a->pt_stride;
  const int64_t row0 = a->q_indptr[r];
  const char* qr = (const char*)a->q + row0 * Hq * d * q_elem_bytes(a->dtype);
  double* o = a->o + row0 * Hq * d;
  double* lse = a->lse + row0 * Hq;
  if (a->is_verify[r]) {
    double* lg = a->logits + a->logits_off[r];
    oracle_verify_request(Hq, Hkv, d, a->sm_scale, a->dtype, L, a->k, qr, a->k_pool, a->v_pool,
                          pt_row, lg, lse, o);
    double* pbar = (double*)malloc(sizeof(double) * (size_t)Hkv * L);
    if (!pbar) return -2;
    oracle_average(Hq, Hkv, L, a->k, a->row_begin, a->row_count, lg, lse, pbar);
    const int K = a->idx_count[r];
    for (int g = 0; g < Hkv; ++g) {
      int rc = oracle_topk(L, K, pbar + (int64_t)g * L, a->idx + a->idx_off[r] + (int64_t)g * K);
      if (rc) {
        free(pbar);
        return rc;
      }
    }
    free(pbar);
  } else {
    oracle_draft_request(Hq, Hkv, d, a->sm_scale, a->dtype, L, qr, a->k_pool, a->v_pool, pt_row,
                         a->idx_count[r], a->idx + a->idx_off[r], o, lse);
  }
  return 0;
}

static void* step_worker(void* p) {
  step_args* a = (step_args*)p;
  for (;;) {
    pthread_mutex_lock(&a->lock);
    int r = a->next++;
    pthread_mutex_unlock(&a->lock);
    if (r >= a->B) break;
    if (a->selected && !a->selected[r]) continue;
    int rc = run_request(a, r);
    if (rc) {
      pthread_mutex_lock(&a->lock);
      a->status = rc;
      pthread_mutex_unlock(&a->lock);
    }
  }
  return NULL;
}

/* Requests are independent, so `nthreads` workers take them one at a time. */
int oracle_step(int B, int k, int Hq, int Hkv, int d, double sm_scale, int dtype,
                int row_begin, int row_count, const uint8_t* is_verify, const int32_t* seq_lens,
                const int32_t* q_indptr, const int32_t* page_table, int64_t pt_stride,
                const void* q, const void* k_pool, const void* v_pool, const int32_t* idx_count,
                const int64_t* idx_off, int32_t* idx, double* o, double* lse, double* logits,
                const int64_t* logits_off, const uint8_t* selected, int nthreads) {
  if (Hkv <= 0 || Hq % Hkv != 0) return -1;
  step_args a;
  memset(&a, 0, sizeof a);
  a.B = B; a.k = k; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.dtype = dtype;
  a.row_begin = row_begin; a.row_count = row_count; a.sm_scale = sm_scale;
  a.is_verify = is_verify; a.seq_lens = seq_lens; a.q_indptr = q_indptr;
  a.page_table = page_table; a.pt_stride = pt_stride; a.q = q; a.k_pool = k_pool;
  a.v_pool = v_pool; a.idx_count = idx_count; a.idx_off = idx_off; a.idx = idx; a.o = o;
  a.lse = lse; a.logits = logits; a.logits_off = logits_off; a.selected = selected;
  pthread_mutex_init(&a.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, step_worker, &a);
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&a.lock);
  return a.status;
}

/* ---- recallable sparse index of one KV head --------------------------------
 * Position j in [0, L) belongs to the index when it is a sink (j < n_sink), a
 * recent token (j >= L - n_recent), or an entry of the stored list `in`
 * (entries outside [0, L) name no position).  Members go to out[0..u)
 * ascending; out[u..cap) is filled with -1, an entry that draft attention
 * ignores.  Returns u, or -1 when u > cap.
 */
int oracle_recall_index(int L, int n_sink, int n_recent, int n_in, const int32_t* in, int cap,
                        int32_t* out) {
  unsigned char* member = (unsigned char*)calloc((size_t)(L > 0 ? L : 1), 1);
  if (!member) return -2;
  for (int j = 0; j < L; ++j) {
    int sink = MUT(15) ? (j <= n_sink) : (j < n_sink);
    int recent = MUT(13) ? (j >= L - n_recent - 1 && j < L - 1) : (j >= L - n_recent);
    if (sink || recent) member[j] = 1;
  }
  for (int t = 0; t < n_in; ++t) {
    int32_t p = in[t];
    if (MUT(14) && p >= L) p = L - 1;
    if (p >= 0 && p < L) member[p] = 1;
  }
  int u = 0;
  for (int j = 0; j < L; ++j) {
    if (!member[j]) continue;
    if (u < cap) out[u] = j;
    ++u;
  }
  free(member);
  if (u > cap) return -1;
  for (int t = u; t < cap; ++t) out[t] = MUT(16) ? 0 : -1;
  return u;
}

/* ---- quality of an index list for one query row -----------------------------
 * logits [Hq][L] (-inf where hidden) and lse [Hq] of the row; list [Hkv][n]
 * positions per KV head (entries outside [0, L) name no position, repeats
 * count once).  Query head h reads the list of KV head h / G, with softmax
 * p_h[j] = exp(logits[h][j] - lse[h]):
 *   coverage[h] = sum of p_h over the list's distinct valid positions;
 *   top[h][0..T) = the T positions of largest p_h (ties to the lower
 *                  position), ascending;
 *   recall[h]   = |top[h] intersected with the list| / T.
 * Returns 0, or -1 when T is not in [1, L].
 */
int oracle_list_quality(int Hq, int Hkv, int L, const double* logits, const double* lse, int n,
                        const int32_t* list, int T, int32_t* top, double* coverage,
                        double* recall) {
  if (T < 1 || T > L) return -1;
  const int G = Hq / Hkv;
  unsigned char* member = (unsigned char*)malloc((size_t)L);
  double* p = (double*)malloc(sizeof(double) * (size_t)L);
  if (!member || !p) {
    free(member);
    free(p);
    return -2;
  }
  for (int h = 0; h < Hq; ++h) {
    const int g = MUT(3) ? h % Hkv : h / G;
    memset(member, 0, (size_t)L);
    for (int t = 0; t < n; ++t) {
      const int32_t pos = list[(int64_t)g * n + t];
      if (pos >= 0 && pos < L) member[pos] = 1;
    }
    double cov = 0.0;
    for (int j = 0; j < L; ++j) {
      const double l = logits[(int64_t)h * L + j];
      p[j] = (l == -INFINITY) ? 0.0 : exp(l - (MUT(17) ? 0.0 : lse[h]));
    }
    if (MUT(18)) {
      for (int t = 0; t < n; ++t) {
        const int32_t pos = list[(int64_t)g * n + t];
        if (pos >= 0 && pos < L) cov += p[pos];
      }
    } else {
      for (int j = 0; j < L; ++j)
        if (member[j]) cov += p[j];
    }
    coverage[h] = cov;
    int32_t* th = top + (int64_t)h * T;
    if (oracle_topk(L, T, p, th)) {
      free(member);
      free(p);
      return -2;
    }
    int hits = 0;
    for (int t = 0; t < T; ++t) hits += member[th[t]];
    recall[h] = (double)hits / (double)T;
  }
  free(member);
  free(p);
  return 0;
}

int oracle_mutant_id(void) { return ORACLE_MUTANT; }
