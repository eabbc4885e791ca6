// sched.cpp -- the host-side scheduler of include/spa_sched.h: phase buckets,
// delayed verification and the per-step batch metadata of spa_unified_step.
//
// Review of SparseSpec, 核心方法 / "Unified batch scheduler + fused attention
// kernel" (requests counted per phase in buckets, new requests to the
// emptiest one) and "Delayed verification" (a verify is issued one step
// late); blog sections 4.2-4.3.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>

#include "spa.h"
#include "spa_error.h"
#include "spa_sched.h"

namespace {

constexpr uint64_t SCHED_MAGIC = 0x5350415343484544ull;  // "SPASCHED"

size_t align64(size_t x) { return (x + 63) / 64 * 64; }

// splitmix64 at a counter: a seeded stream of independent 64-bit draws.
uint64_t mix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

// State layout: this header, then the arrays at the offsets it records.
struct Header {
  uint64_t magic;
  spa_sched_config cfg;
  int32_t cycle;      // C: k+1, or k+2 with delayed verification
  int32_t k_cap;      // list entries per KV head a slot can hold: ceil(s max_len)
  int32_t planned;    // 1 between spa_sched_next and spa_sched_commit
  int64_t step;
  uint64_t draws;     // random draws taken
  spa_sched_stats stats;
  int32_t n_new;
  int32_t pad_;
  // per slot
  size_t bucket, ctx, target, produced, k_last, lead;
  // per step
  size_t is_verify, seq_lens, q_indptr, idx_count, idx_off, logits_off, slot, role;
  size_t new_slots, new_len, new_count;
  size_t counts;  // [cycle]
  size_t total;
};

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}
template <typename T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

int64_t ceil_frac(int64_t L, int32_t num, int32_t den) { return (L * num + den - 1) / den; }

int32_t check_config(const spa_sched_config* c) {
  if (!c) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler config is NULL");
  if (c->slots < 1) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: slots < 1");
  if (c->spec_k < 1 || c->spec_k > 64) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: spec_k outside [1, 64]");
  if (c->num_qo_heads < 1 || c->num_kv_heads < 1 || c->num_qo_heads % c->num_kv_heads != 0)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: head counts");
  if (c->sparsity_num < 1 || c->sparsity_den < c->sparsity_num)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: sparsity must lie in (0, 1]");
  if (c->prompt_min <= c->spec_k || c->prompt_max < c->prompt_min)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: prompt range (prompt_min must exceed spec_k)");
  if (c->output_min < 1 || c->output_max < c->output_min)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: output range");
  if ((int64_t)c->prompt_max + c->output_max + c->spec_k + 1 > c->max_len)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: prompt_max + output_max + spec_k + 1 exceeds max_len");
  if (!(c->accept_prob >= 0.f && c->accept_prob <= 1.f))
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: accept_prob outside [0, 1]");
  return SPA_OK;
}

Header layout(const spa_sched_config& c) {
  Header h;
  std::memset(&h, 0, sizeof h);
  h.cfg = c;
  h.cycle = c.spec_k + 1 + (c.delayed ? 1 : 0);
  h.k_cap = (int32_t)ceil_frac(c.max_len, c.sparsity_num, c.sparsity_den);
  const size_t S = (size_t)c.slots;
  size_t o = align64(sizeof(Header));
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = align64(o + bytes);
    return r;
  };
  h.bucket = take(S * 4);
  h.ctx = take(S * 4);
  h.target = take(S * 4);
  h.produced = take(S * 4);
  h.k_last = take(S * 4);
  h.lead = take(S * 4);
  h.is_verify = take(S);
  h.seq_lens = take(S * 4);
  h.q_indptr = take((S + 1) * 4);
  h.idx_count = take(S * 4);
  h.idx_off = take(S * 8);
  h.logits_off = take(S * 8);
  h.slot = take(S * 4);
  h.role = take(S * 4);
  h.new_slots = take(S * 4);
  h.new_len = take(S * 4);
  h.new_count = take(S * 4);
  h.counts = take((size_t)h.cycle * 4);
  h.total = o;
  return h;
}

uint64_t draw(Header* h) { return mix64(h->cfg.seed * 0x632be59bd9b4e019ull + h->draws++); }

int32_t uniform_int(Header* h, int32_t lo, int32_t hi) {  // [lo, hi]
  return lo + (int32_t)(draw(h) % (uint64_t)(hi - lo + 1));
}

// A new request in slot s, first planned at step t: its prompt, its target
// and the emptiest bucket.  The bucket's phase at step t is ph; the request
// joins it there, so its first cycle has only k - j0 draft steps left (j0 =
// ph for a draft or the verify phase, 0 for the skipped phase after a delayed
// verify).  Its first verify still has k+1 rows: they start j0 positions
// before the pending token (the last j0 prompt tokens are checked again and
// count as accepted), so its committed length starts at P - j0 and the first
// step it is issued in has context P + 1 whatever its phase.
void admit(void* st, Header* h, int32_t s, int64_t t) {
  const spa_sched_config& c = h->cfg;
  int32_t* counts = at<int32_t>(st, h->counts);
  int32_t b = 0;
  for (int32_t i = 1; i < h->cycle; ++i)
    if (counts[i] < counts[b]) b = i;
  counts[b] += 1;
  at<int32_t>(st, h->bucket)[s] = b;
  const int32_t ph = (int32_t)((t + b) % h->cycle);
  const int32_t j0 = ph <= c.spec_k ? ph : 0;
  const int32_t P = uniform_int(h, c.prompt_min, c.prompt_max);
  at<int32_t>(st, h->ctx)[s] = P - j0;
  at<int32_t>(st, h->lead)[s] = j0;
  at<int32_t>(st, h->target)[s] = uniform_int(h, c.output_min, c.output_max);
  at<int32_t>(st, h->produced)[s] = 0;
  const int32_t K0 = (int32_t)ceil_frac(P, c.sparsity_num, c.sparsity_den);
  at<int32_t>(st, h->k_last)[s] = K0;
  const int32_t n = h->n_new++;
  at<int32_t>(st, h->new_slots)[n] = s;
  at<int32_t>(st, h->new_len)[n] = P;
  at<int32_t>(st, h->new_count)[n] = K0;
}

Header* header(void* st) {
  Header* h = static_cast<Header*>(st);
  return (h && h->magic == SCHED_MAGIC) ? h : nullptr;
}
const Header* header(const void* st) {
  const Header* h = static_cast<const Header*>(st);
  return (h && h->magic == SCHED_MAGIC) ? h : nullptr;
}

enum Role : int32_t { ROLE_WAIT = 0, ROLE_DRAFT = 1, ROLE_VERIFY = 2 };

}  // namespace

extern "C" {

size_t spa_sched_bytes(const spa_sched_config* cfg) {
  if (check_config(cfg)) return 0;
  return layout(*cfg).total;
}

int32_t spa_sched_capacity(const spa_sched_config* cfg, int64_t* idx_elems, int64_t* logits_elems,
                           int32_t* rows) {
  const int32_t rc = check_config(cfg);
  if (rc) return rc;
  const Header h = layout(*cfg);
  const int64_t S = cfg->slots, k = cfg->spec_k;
  if (idx_elems) *idx_elems = S * cfg->num_kv_heads * h.k_cap;
  // at most ceil(S / C) + 1 requests share a phase (buckets stay within one)
  const int64_t nv = std::min<int64_t>(S, (S + h.cycle - 1) / h.cycle + 1);
  if (logits_elems) *logits_elems = nv * (k + 1) * cfg->num_qo_heads * cfg->max_len;
  if (rows) *rows = (int32_t)(S + nv * k);
  return SPA_OK;
}

int32_t spa_sched_init(void* state, size_t bytes, const spa_sched_config* cfg) {
  int32_t rc = check_config(cfg);
  if (rc) return rc;
  if (!state) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state is NULL");
  if ((reinterpret_cast<uintptr_t>(state) & 63) != 0)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state must be 64-byte aligned");
  const Header h0 = layout(*cfg);
  if (bytes < h0.total)
    return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state of " + std::to_string(bytes) +
                                                   " bytes, need " + std::to_string(h0.total));
  std::memset(state, 0, h0.total);
  Header* h = static_cast<Header*>(state);
  *h = h0;
  h->magic = SCHED_MAGIC;
  for (int32_t s = 0; s < cfg->slots; ++s) admit(state, h, s, 0);
  return SPA_OK;
}

int32_t spa_sched_next(void* state, spa_sched_step* out) {
  Header* h = header(state);
  if (!h || !out) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state not initialised or out is NULL");
  const spa_sched_config& c = h->cfg;
  const int32_t k = c.spec_k;
  uint8_t* is_verify = at<uint8_t>(state, h->is_verify);
  int32_t* seq_lens = at<int32_t>(state, h->seq_lens);
  int32_t* q_indptr = at<int32_t>(state, h->q_indptr);
  int32_t* idx_count = at<int32_t>(state, h->idx_count);
  int64_t* idx_off = at<int64_t>(state, h->idx_off);
  int64_t* logits_off = at<int64_t>(state, h->logits_off);
  int32_t* slot = at<int32_t>(state, h->slot);
  int32_t* role = at<int32_t>(state, h->role);
  const int32_t* bucket = at<int32_t>(state, h->bucket);
  const int32_t* ctx = at<int32_t>(state, h->ctx);
  const int32_t* k_last = at<int32_t>(state, h->k_last);
  int32_t B = 0, rows = 0, nv = 0, nd = 0, nw = 0;
  int64_t lg = 0;
  for (int32_t s = 0; s < c.slots; ++s) {
    const int32_t ph = (int32_t)((h->step + bucket[s]) % h->cycle);
    if (ph < k) {
      role[s] = ROLE_DRAFT;
      slot[B] = s;
      q_indptr[B] = rows;
      is_verify[B] = 0;
      seq_lens[B] = ctx[s] + ph + 1;
      idx_count[B] = k_last[s];
      logits_off[B] = 0;
      rows += 1;
      nd += 1;
    } else if (ph == k) {
      role[s] = ROLE_VERIFY;
      const int32_t L = ctx[s] + k + 1;
      slot[B] = s;
      q_indptr[B] = rows;
      is_verify[B] = 1;
      seq_lens[B] = L;
      idx_count[B] = (int32_t)ceil_frac(L, c.sparsity_num, c.sparsity_den);
      logits_off[B] = lg;
      lg += (int64_t)(k + 1) * c.num_qo_heads * L;
      rows += k + 1;
      nv += 1;
    } else {
      role[s] = ROLE_WAIT;
      nw += 1;
      continue;
    }
    idx_off[B] = (int64_t)s * c.num_kv_heads * h->k_cap;
    B += 1;
  }
  q_indptr[B] = rows;
  h->planned = 1;
  out->step = h->step;
  out->B = B;
  out->rows = rows;
  out->n_verify = nv;
  out->n_draft = nd;
  out->n_waiting = nw;
  out->n_new = h->n_new;
  out->is_verify = is_verify;
  out->seq_lens = seq_lens;
  out->q_indptr = q_indptr;
  out->idx_count = idx_count;
  out->idx_off = idx_off;
  out->logits_off = logits_off;
  out->slot = slot;
  out->new_slots = at<int32_t>(state, h->new_slots);
  out->new_len = at<int32_t>(state, h->new_len);
  out->new_count = at<int32_t>(state, h->new_count);
  out->logits_elems = lg;
  return SPA_OK;
}

int32_t spa_sched_commit(void* state) {
  Header* h = header(state);
  if (!h) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state not initialised");
  if (!h->planned) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: commit without a planned step");
  const spa_sched_config& c = h->cfg;
  const int32_t k = c.spec_k;
  const int32_t* role = at<int32_t>(state, h->role);
  int32_t* ctx = at<int32_t>(state, h->ctx);
  int32_t* produced = at<int32_t>(state, h->produced);
  int32_t* k_last = at<int32_t>(state, h->k_last);
  int32_t* lead = at<int32_t>(state, h->lead);
  const int32_t* target = at<int32_t>(state, h->target);
  int32_t* bucket = at<int32_t>(state, h->bucket);
  int32_t* counts = at<int32_t>(state, h->counts);
  h->n_new = 0;
  for (int32_t s = 0; s < c.slots; ++s) {
    if (role[s] == ROLE_DRAFT) {
      h->stats.drafts += 1;
      h->stats.rows += 1;
      continue;
    }
    if (role[s] == ROLE_WAIT) {
      h->stats.waits += 1;
      continue;
    }
    // a verify: the leading run of accepted drafts, then one more token; the
    // first j0 rows of a new request's first verify are prompt tokens
    const int32_t L = ctx[s] + k + 1;
    const int32_t j0 = lead[s];
    int32_t a = 0;
    while (a < k - j0) {
      const double u = (double)(draw(h) >> 11) * (1.0 / 9007199254740992.0);
      if (!(u < (double)c.accept_prob)) break;
      ++a;
    }
    k_last[s] = (int32_t)ceil_frac(L, c.sparsity_num, c.sparsity_den);
    ctx[s] += j0 + a + 1;
    produced[s] += a + 1;
    lead[s] = 0;
    h->stats.verifies += 1;
    h->stats.drafted += k - j0;
    h->stats.accepted += a;
    h->stats.committed += a + 1;
    h->stats.rows += k + 1;
    if (produced[s] >= target[s]) {
      counts[bucket[s]] -= 1;
      h->stats.retired += 1;
      admit(state, h, s, h->step + 1);
    }
  }
  h->stats.steps += 1;
  h->step += 1;
  h->planned = 0;
  return SPA_OK;
}

int32_t spa_sched_stats_read(const void* state, spa_sched_stats* out) {
  const Header* h = header(state);
  if (!h || !out) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state not initialised or out is NULL");
  *out = h->stats;
  return SPA_OK;
}

int32_t spa_sched_buckets(const void* state, int32_t* counts, int32_t n) {
  const Header* h = header(state);
  if (!h || !counts) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler state not initialised or counts is NULL");
  if (n < h->cycle) return spa::set_error(SPA_ERR_INVALID_ARG, "scheduler: counts holds fewer than the cycle's phases");
  std::memcpy(counts, at<int32_t>(state, h->counts), (size_t)h->cycle * 4);
  return SPA_OK;
}

}  // extern "C"
