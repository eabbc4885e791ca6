// api.cpp -- host side of libspa: argument checks, work planning and kernel
// launches behind the C ABI of include/spa.h.
//
// A call turns the host metadata into a work plan -- one record per workgroup
// -- written into the caller's pinned plan buffer, which the kernels read in
// place (no copy is enqueued).  The attention plan lists its items longest
// first; persistent attention workgroups draw the next item from a work
// counter in the caller's workspace, so work flows to whichever XCD frees
// first.  A call enqueues at most three launches: the attention of every
// request, the post-pass (split-K merges and score averaging), then the top-K
// selection.  The library holds no per-call state: a plan buffer's header
// carries the release protocol that tells a later call when the GPU no longer
// reads it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "spa.h"
#include "spa_error.h"
#include "spa_kernels.h"
#include "spa_plan.h"

using namespace spa;

namespace {
thread_local std::string g_err;
}  // namespace

int32_t spa::set_error(int32_t code, const std::string& msg) {
  g_err = msg;
  return code;
}

namespace {

constexpr int DEFAULT_VERIFY_CHUNK = 2048;  // fewer split-K partials
constexpr int MIN_AUTO_VERIFY_CHUNK = 512;
constexpr int DEFAULT_DRAFT_CHUNK = 1024;
constexpr int DEFAULT_CUS = 256;  // MI355X

int32_t fail(int32_t code, const std::string& msg) {
  g_err = msg;
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Req {
  int32_t L = 0;
  int32_t pt_row = 0;  // page-table row
  bool verify = false;
  int32_t row0 = 0;
  int32_t nlist = 0;  // draft: entries per KV head; verify: K_r
  int64_t logits_off = 0;
  int64_t idx_off = 0;
};

struct Shape {
  int Hq = 0, Hkv = 0, G = 0, d = 0, dtype = 0, k = 0;
  int64_t num_slots = 0;
  int32_t stride = 0;
  float scale = 0.f;
};

// A call's work plan.  plan_size() fixes every count, offset and the item
// order; plan_write() then writes the records straight into the pinned slot,
// so the host touches each record once.
struct Plan {
  bool attn = false, topk = false;
  std::vector<int32_t> order;   // requests by estimated bytes, descending
  std::vector<int32_t> nchunk;  // split-K chunks of request r
  std::vector<int64_t> part0;   // first split-K partial row of (r, 0); heads follow
  int max_nchunk = 1;           // most split-K chunks of any merged request
  int cv = DEFAULT_VERIFY_CHUNK;  // positions per verify item
  int cd = DEFAULT_DRAFT_CHUNK;   // list entries per draft item
  int ng = 1;                   // KV heads per item of an unsplit draft request (MFMA path)
  int n_items = 0;              // attention records
  // split: a mixed batch runs its draft items in a second attention launch on
  // a side stream, concurrently with verify attention, merge, averaging and
  // top-K on the caller's stream
  bool split = false;
  int n_items_d = 0;            // draft launch records
  int n_merge_d = 0;            // draft merges, run after the join
  int n_merge = 0, n_avg = 0, n_sel = 0;
  int n_hist = 0;  // selected rows with a score histogram (all of them when the call has attention)
  int max_sel_len = 0;  // longest selected row
  int max_row_sel_len = 0;  // longest row selected by one workgroup
  int n_chunks = 0;  // chunks of the long rows selected in chunks (sel_chunked)
  int n_chunked_rows = 0;  // selected rows of those
  int64_t part_rows = 0;
  int64_t pbar_elems = 0;
  int64_t avg_logit_bytes = 0;  // logits the verify requests dump, which the averaging reads back
  // pinned plan layout
  size_t h_items = 0, h_items_d = 0, h_post = 0, h_post_d = 0, h_sel = 0, h_chunks = 0, h_bytes = 0;
  // workspace layout (work counters at offset 0)
  size_t off_part_o = 0, off_part_ml = 0, off_pbar = 0, off_plan = 0, off_hist = 0, total = 0;
  // chunked long-row selection: row boundaries, each chunk's counts above and
  // in the boundary bin, each chunk's candidates
  size_t hist_zero_bytes = 0, off_row_info = 0, off_cnt_above = 0, off_cnt_bin = 0, off_cand_key = 0,
         off_cand_pos = 0;
  int nthr = 256;
  size_t smem = 0;
};

// The options a call uses (spa_options with its defaults applied).
struct Opts {
  int verify_chunk = 0;  // 0: automatic
  int draft_chunk = DEFAULT_DRAFT_CHUNK;
  int num_cus = DEFAULT_CUS;
  bool overlap = false;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t timing[8] = {};
  const int32_t* pt_rows = nullptr;  // page-table row of each request (null: row r)
  int32_t pt_row_count = 0;
};

int32_t check_opts(const spa_options* o, Opts* out) {
  *out = Opts{};
  if (!o) return SPA_OK;
  if (o->verify_chunk < 0 || o->verify_chunk > VERIFY_MAX_CHUNK)
    return fail(SPA_ERR_INVALID_ARG, "options: verify_chunk outside [0, 2048]");
  if (o->draft_chunk < 0 || o->draft_chunk > DRAFT_MAX_CHUNK)
    return fail(SPA_ERR_INVALID_ARG, "options: draft_chunk outside [0, 2048]");
  if (o->num_cus < 0) return fail(SPA_ERR_INVALID_ARG, "options: num_cus < 0");
  out->verify_chunk = o->verify_chunk;
  if (o->draft_chunk > 0) out->draft_chunk = o->draft_chunk;
  if (o->num_cus > 0) out->num_cus = o->num_cus;
  out->overlap = o->overlap != 0;
  out->side = static_cast<hipStream_t>(o->side_stream);
  out->fork = static_cast<hipEvent_t>(o->fork_event);
  out->join = static_cast<hipEvent_t>(o->join_event);
  for (int i = 0; i < 8; ++i) out->timing[i] = static_cast<hipEvent_t>(o->timing[i]);
  out->pt_rows = o->page_table_rows;
  out->pt_row_count = o->page_table_row_count;
  if (out->pt_rows && out->pt_row_count < 1)
    return fail(SPA_ERR_INVALID_ARG, "options: page_table_row_count must be positive");
  return SPA_OK;
}



// Page-table row of each request: options.page_table_rows[r] (checked
// against the row count) or r.
int32_t apply_pt_rows(const Opts& o, std::vector<Req>* rq) {
  for (size_t r = 0; r < rq->size(); ++r) {
    const int32_t x = o.pt_rows ? o.pt_rows[r] : (int32_t)r;
    if (o.pt_rows && (x < 0 || x >= o.pt_row_count))
      return fail(SPA_ERR_INVALID_ARG, "options: page_table_rows[" + std::to_string(r) +
                                           "] outside [0, " + std::to_string(o.pt_row_count) + ")");
    (*rq)[r].pt_row = x;
  }
  return SPA_OK;
}

int32_t check_layout(const spa_layout* lay, Shape* s) {
  if (!lay) return fail(SPA_ERR_INVALID_ARG, "layout is NULL");
  if (lay->num_qo_heads <= 0 || lay->num_kv_heads <= 0)
    return fail(SPA_ERR_INVALID_ARG, "head counts must be positive");
  if (lay->num_qo_heads % lay->num_kv_heads != 0)
    return fail(SPA_ERR_INVALID_ARG, "num_qo_heads must be a multiple of num_kv_heads");
  if (lay->num_kv_heads > 255) return fail(SPA_ERR_UNSUPPORTED, "num_kv_heads above 255");
  if (lay->head_dim != 64 && lay->head_dim != 128)
    return fail(SPA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (lay->dtype != SPA_BF16 && lay->dtype != SPA_F32)
    return fail(SPA_ERR_UNSUPPORTED, "dtype must be SPA_BF16 or SPA_F32");
  if (lay->num_slots <= 0) return fail(SPA_ERR_INVALID_ARG, "num_slots must be positive");
  if (lay->num_slots > 0x7fffffffLL) return fail(SPA_ERR_UNSUPPORTED, "num_slots above 2^31-1");
  if (lay->page_table_stride <= 0)
    return fail(SPA_ERR_INVALID_ARG, "page_table_stride must be positive");
  if (!(lay->sm_scale >= 0.f) || std::isinf(lay->sm_scale))
    return fail(SPA_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
  s->Hq = lay->num_qo_heads;
  s->Hkv = lay->num_kv_heads;
  s->G = s->Hq / s->Hkv;
  s->d = lay->head_dim;
  s->dtype = lay->dtype;
  s->num_slots = lay->num_slots;
  s->stride = lay->page_table_stride;
  s->scale = lay->sm_scale > 0.f ? lay->sm_scale : 1.f / std::sqrt((float)lay->head_dim);
  return SPA_OK;
}

// Segments [off, off+len) must be non-negative and pairwise disjoint.
int32_t check_segments(std::vector<std::pair<int64_t, int64_t>> seg, const char* what) {
  for (auto& x : seg)
    if (x.first < 0) return fail(SPA_ERR_INVALID_ARG, std::string(what) + ": negative offset");
  std::sort(seg.begin(), seg.end());
  for (size_t i = 1; i < seg.size(); ++i)
    if (seg[i - 1].first + seg[i - 1].second > seg[i].first)
      return fail(SPA_ERR_INVALID_ARG, std::string(what) + ": overlapping segments");
  return SPA_OK;
}

// Positions per verify item.  Unless set in the options: the longest of 2048,
// 1536 and 1024 positions that still gives the verify requests at least two
// items per resident attention workgroup (two per CU when a workgroup has at
// most four waves, that is at most 48 query rows per KV head on the MFMA
// path; one otherwise), else 512.  Long chunks need fewer split-K partials and
// merges; enough items let workgroups that finish early take more, which
// shortens the launch's tail.  Measured (steady state, same box): Qwen3-8B
// shape 179.5 us at 512 (640: 182.9, 768: 186.9, 1024: 192.2), Qwen3-14B
// shape best at 2048, long context 294.1 us at 2048 and 289.5 at 1536; the
// rule picks 512, 2048 and 1536 for them.  Only the verify requests count, so
// a verify-only call and a mixed one split alike.
int verify_chunk(const std::vector<Req>& rq, int Hkv, int rows_v, int G, bool bf16, const Opts& o) {
  if (o.verify_chunk > 0) return o.verify_chunk;
  int longest = 0;
  for (const Req& q : rq)
    if (q.verify) longest = std::max(longest, q.L);
  const int64_t slots = (int64_t)o.num_cus * ((bf16 && rows_v * G > 48) ? 1 : 2);
  auto items = [&](int c) {
    int64_t n = 0;
    for (const Req& q : rq)
      if (q.verify) n += (int64_t)((q.L + c - 1) / c) * Hkv * (bf16 ? 1 : rows_v);
    return n;
  };
  int c = MIN_AUTO_VERIFY_CHUNK;
  for (const int cand : {DEFAULT_VERIFY_CHUNK, 1536, 1024})
    if (items(cand) >= 2 * slots) {
      c = cand;
      break;
    }
  // a request may not need more split-K chunks than a merge takes
  while (c < DEFAULT_VERIFY_CHUNK && (longest + c - 1) / c > MAX_MERGE_CHUNKS)
    c = std::min(2 * c, DEFAULT_VERIFY_CHUNK);
  return c;
}

int avg_parts(int L) { return (L + AVG_SPAN - 1) / AVG_SPAN; }
int64_t pbar_row(int L) { return (L + 3) / 4 * 4; }  // rows start 16-byte aligned

// Counts, offsets and the item order of the attention (attn) and/or PillarAttn
// selection (topk) plan for `rq`.
int32_t plan_size(const Shape& s, const std::vector<Req>& rq, bool attn, bool topk, const Opts& o,
                  Plan* pl) {
  const int B = (int)rq.size();
  const int G = s.G, Hkv = s.Hkv, D = s.d;
  const int rows_v = s.k + 1;
  const bool bf16 = s.dtype == SPA_BF16;
  const int esz = bf16 ? 2 : 4;
  const int CV = verify_chunk(rq, Hkv, s.k + 1, G, s.dtype == SPA_BF16, o), CD = o.draft_chunk;
  pl->cv = CV;
  pl->cd = CD;
  if (s.k > 255) return fail(SPA_ERR_UNSUPPORTED, "spec_k above 255");
  pl->attn = attn;
  pl->topk = topk;

  bool any_verify = false, any_draft = false;
  for (auto& q : rq) (q.verify ? any_verify : any_draft) = true;
  pl->split = attn && topk && any_verify && any_draft && o.overlap;
  if (pl->split && (!o.side || !o.fork || !o.join))
    return fail(SPA_ERR_INVALID_ARG, "options: overlap needs side_stream, fork_event and join_event");

  pl->nchunk.assign(B, 1);
  pl->part0.assign(B, 0);
  int64_t part_rows = 0;
  if (attn) {
    // Packed drafts (MFMA path): an unsplit draft request's KV heads go ng to
    // an item, so that an item's startup (record, list and page-table reads,
    // first tile: about 8 us at load) is paid once per ng lists.  Packing
    // doubles ng while the lists are short (ng times the longest one's tiles
    // at most PACK_TILES), the slots and the staged query rows fit LDS, and
    // the draft items still number two per CU in a draft-only call, or one
    // per CU beside verify items, which keep the other workgroups busy
    // (measured: the Qwen3-8B-shaped mixed step 182.6 -> 181.8 us, draft-only
    // batches unchanged).
    if (bf16) {
      int64_t lists = 0;
      int tiles = 0;
      for (const Req& q : rq)
        if (!q.verify && q.nlist <= CD) {
          lists += Hkv;
          tiles = std::max(tiles, (q.nlist + TILE_TOKENS - 1) / TILE_TOKENS);
        }
      while (lists > 0 && Hkv % (2 * pl->ng) == 0 && 2 * pl->ng * tiles <= PACK_TILES &&
             lists / (2 * pl->ng) >= (any_verify ? 1 : 2) * (int64_t)o.num_cus &&
             2 * pl->ng * tiles * TILE_TOKENS <= VERIFY_MAX_CHUNK &&
             2 * pl->ng * G * D * esz <= PACK_Q_BYTES)
        pl->ng *= 2;
    }
    std::vector<double> bytes(B);
    std::vector<int> nitems(B);
    for (int r = 0; r < B; ++r) {
      const Req& q = rq[r];
      const bool v = q.verify;
      const int span = v ? q.L : q.nlist;
      const int chunk = v ? CV : CD;
      const int nc = std::max(1, (span + chunk - 1) / chunk);
      if (nc > MAX_MERGE_CHUNKS) return fail(SPA_ERR_UNSUPPORTED, "more than 256 split-K chunks per request");
      pl->nchunk[r] = nc;
      if (nc > 1) pl->max_nchunk = std::max(pl->max_nchunk, nc);
      nitems[r] = nc * ((v && !bf16) ? rows_v : 1);  // fp32 verify: one item per query row
      if (!v && nc == 1 && pl->ng > 1) nitems[r] = -pl->ng;  // ng KV heads per item
      if (nc > 1) {
        pl->part0[r] = part_rows;
        part_rows += (int64_t)Hkv * nc * (v ? rows_v : 1) * G;
        const int nm = Hkv * ((((v ? rows_v : 1) * G) + MERGE_ROWS - 1) / MERGE_ROWS);
        if (pl->split && !v)
          pl->n_merge_d += nm;
        else
          pl->n_merge += nm;
      }
      const double head_bytes = v ? (double)q.L * (2.0 * D * esz + 4 + 4.0 * rows_v * G)
                                  : (double)q.nlist * (2.0 * D * esz + 8);
      bytes[r] = nitems[r] < 0 ? head_bytes * -nitems[r] : head_bytes / nitems[r];  // per item
    }
    // persistent workgroups draw items in record order, so the records go
    // longest first: requests by their items' estimated bytes (all items of a
    // request weigh about the same), each request's items together.  Ordered
    // by whole requests instead, packed draft items (two lists) went after the
    // shorter verify chunks: the Qwen3-8B-shaped step 181.4 -> 179.7 us by item.
    pl->order.resize(B);
    for (int r = 0; r < B; ++r) pl->order[r] = r;
    std::stable_sort(pl->order.begin(), pl->order.end(),
                     [&](int a, int b) { return bytes[a] > bytes[b]; });
    for (int r = 0; r < B; ++r)
      ((pl->split && !rq[r].verify) ? pl->n_items_d : pl->n_items) +=
          nitems[r] < 0 ? Hkv / -nitems[r] : Hkv * nitems[r];
  }
  int64_t pbar = 0;
  if (topk)
    for (auto& q : rq)
      if (q.verify) {
        pl->n_avg += Hkv * avg_parts(q.L);
        pl->avg_logit_bytes += (int64_t)q.L * s.Hq * 4 * (s.k + 1);
        pl->n_sel += Hkv;
        pl->max_sel_len = std::max(pl->max_sel_len, q.L);
        // the histogram is cleared by the attention launch, so only a call
        // with one keeps it
        if (attn) pl->n_hist += Hkv;
        if (attn && sel_chunked(q.L)) {
          pl->n_chunks += Hkv * ((q.L + SELECT_SPAN - 1) / SELECT_SPAN);
          pl->n_chunked_rows += Hkv;
        }
        else
          pl->max_row_sel_len = std::max(pl->max_row_sel_len, q.L);
        pbar += Hkv * pbar_row(q.L);
      }
  pl->part_rows = part_rows;
  pl->pbar_elems = pbar;

  // block shape and LDS of the attention launch
  // bf16: every item on the MFMA path; fp32: every item on the VALU path
  bool need_mfma = false, need_valu = false;
  if (attn) {
    need_mfma = bf16;
    need_valu = !bf16;
  }
  int nthr = 256;
  if (need_mfma) {
    const int nt = ((any_verify ? rows_v : 1) * G + 15) / 16;
    if (nt > MAX_ROW_TILES)
      return fail(SPA_ERR_UNSUPPORTED, "(k+1)*G above 112 rows per KV head on the MFMA path");
    nthr = 64 * std::max(4, nt + 1);  // one consumer wave per row tile, one producer wave
  }
  if (need_valu && G > MAX_GROUP)
    return fail(SPA_ERR_UNSUPPORTED, "GQA group above 8 on the fp32 path");
  pl->nthr = nthr;
  // LDS slot entries of the longest item: positions (verify) or list entries
  // (draft; a packed item's lists each padded to whole tiles, then its query
  // rows, two bf16 per entry)
  int max_chunk = 1;
  for (auto& q : rq) {
    max_chunk = std::max(max_chunk, std::min(q.verify ? q.L : q.nlist, q.verify ? CV : CD));
    if (attn && !q.verify && pl->ng > 1 && q.nlist <= CD)
      max_chunk = std::max(max_chunk, pl->ng * ((q.nlist + TILE_TOKENS - 1) / TILE_TOKENS) * TILE_TOKENS +
                                          pl->ng * G * D * esz / 4);
  }
  pl->smem = attn ? attn_smem_bytes(s.dtype, D, G, nthr, need_mfma, need_valu, max_chunk) : 0;

  // pinned plan layout
  size_t h = 0;
  pl->h_items = h;
  h = align_up(h + (size_t)pl->n_items * sizeof(Item), 256);
  pl->h_items_d = h;
  h = align_up(h + (size_t)pl->n_items_d * sizeof(Item), 256);
  pl->h_post = h;
  h = align_up(h + (size_t)(pl->n_avg + pl->n_merge) * sizeof(PostItem), 256);
  pl->h_post_d = h;
  h = align_up(h + (size_t)pl->n_merge_d * sizeof(PostItem), 256);
  pl->h_sel = h;
  h = align_up(h + (size_t)pl->n_sel * sizeof(PostItem), 256);
  pl->h_chunks = h;  // copied to the workspace with the selection records
  h = align_up(h + (size_t)pl->n_chunks * sizeof(SelChunk), 256);
  pl->h_bytes = h;
  // workspace layout: the attention launches' work counters first
  size_t w = WS_COUNTERS;
  pl->off_part_o = w;  // partial outputs in the output type
  w = align_up(w + (size_t)part_rows * D * esz, 256);
  pl->off_part_ml = w;
  w = align_up(w + (size_t)part_rows * 2 * 4, 256);
  pl->off_pbar = w;
  w = align_up(w + (size_t)pbar * 4, 256);
  // the attention launch (or, without one, the post-pass) copies the records
  // of the launches after it here
  pl->off_plan = w;
  if (attn || topk) w = align_up(w + (pl->h_bytes - pl->h_post), 256);
  pl->off_hist = w;
  w += (size_t)pl->n_hist * HIST_BINS * 4;
  w = align_up(w, 16);
  pl->hist_zero_bytes = w - pl->off_hist;
  w = align_up(w, 256);
  if (pl->n_chunks > 0) {
    pl->off_row_info = w;
    w = align_up(w + (size_t)pl->n_hist * 16, 256);
    pl->off_cnt_above = w;
    w = align_up(w + (size_t)pl->n_chunks * 4, 256);
    pl->off_cnt_bin = w;
    w = align_up(w + (size_t)pl->n_chunks * 4, 256);
    pl->off_cand_key = w;
    w = align_up(w + (size_t)pl->n_chunks * SEL_CAND_CAP * 4, 256);
    pl->off_cand_pos = w;
    w = align_up(w + (size_t)pl->n_chunks * SEL_CAND_CAP * 4, 256);
  }
  pl->total = w;
  return SPA_OK;
}

// Writes the records of a sized plan into the pinned slot at `h`.
void plan_write(const Shape& s, const std::vector<Req>& rq, const Plan& pl, char* h) {
  const int B = (int)rq.size();
  const int G = s.G, Hkv = s.Hkv;
  const int rows_v = s.k + 1;
  const bool bf16 = s.dtype == SPA_BF16;
  const int CV = pl.cv, CD = pl.cd;
  if (pl.attn) {
    Item* items_v = reinterpret_cast<Item*>(h + pl.h_items);
    Item* items_d = reinterpret_cast<Item*>(h + pl.h_items_d);
    int cur_v = 0, cur_dr = 0;
    for (int r : pl.order) {
      const Req& q = rq[r];
      const bool v = q.verify;
      const int span = v ? q.L : q.nlist;
      const int chunk = v ? CV : CD;
      const int nc = pl.nchunk[r];
      const int nq = (v && !bf16) ? rows_v : 1;
      const int64_t head_rows = (int64_t)nc * (v ? rows_v : 1) * G;
      Item* items = (pl.split && !v) ? items_d : items_v;
      int& cur = (pl.split && !v) ? cur_dr : cur_v;
      const int ng = (!v && nc == 1) ? pl.ng : 1;
      for (int g = 0; g < Hkv; g += ng) {
        Item it;
        std::memset(&it, 0, sizeof it);
        it.kind = v ? KIND_VERIFY : KIND_DRAFT;
        it.r = q.pt_row;
        it.g = g;
        it.L = q.L;
        it.row0 = q.row0;
        it.nchunk = nc;
        it.list_len = q.nlist;
        it.off = v ? q.logits_off : q.idx_off + (int64_t)g * q.nlist;
        it.part_row0 = nc > 1 ? pl.part0[r] + g * head_rows : 0;
        it.ng = ng;
        for (int c = 0; c < nc; ++c)
          for (int qi = 0; qi < nq; ++qi) {
            it.qi = qi;
            it.split = c;
            it.begin = c * chunk;
            it.end = std::min(span, (c + 1) * chunk);
            items[cur++] = it;
          }
      }
    }
  }
  // post-pass: the averaging chunks of every verify (r, g), then the split-K
  // merges (measured faster than the reverse order)
  PostItem* post = reinterpret_cast<PostItem*>(h + pl.h_post);
  PostItem* post_d = reinterpret_cast<PostItem*>(h + pl.h_post_d);
  PostItem* sel = reinterpret_cast<PostItem*>(h + pl.h_sel);
  SelChunk* chunks = reinterpret_cast<SelChunk*>(h + pl.h_chunks);
  int nck = 0;
  int np = 0, ns = 0, npd = 0, nh = 0;
  if (pl.topk) {
    int64_t pbar = 0;
    for (int r = 0; r < B; ++r) {
      const Req& q = rq[r];
      if (!q.verify) continue;
      const int nparts = avg_parts(q.L);
      const int nc = pl.attn ? pl.nchunk[r] : 1;
      const int64_t head_rows = (int64_t)nc * rows_v * G;
      for (int g = 0; g < Hkv; ++g) {
        PostItem a;
        std::memset(&a, 0, sizeof a);
        a.kind = POST_AVG;
        a.r = r;
        a.g = g;
        a.rows_q = rows_v;
        a.L = q.L;
        a.row0 = q.row0;
        a.nchunk = nc;
        a.part_row0 = nc > 1 ? pl.part0[r] + g * head_rows : 0;
        a.K = q.nlist;
        a.logits_off = q.logits_off;
        a.idx_off = q.idx_off + (int64_t)g * q.nlist;
        a.pbar_off = pbar;
        a.hist_slot = pl.n_hist > 0 ? nh++ : -1;
        sel[ns++] = a;
        if (pl.n_chunks > 0 && sel_chunked(q.L)) {
          const int first = nck, n = (q.L + SELECT_SPAN - 1) / SELECT_SPAN;
          for (int c = 0; c < n; ++c)
            chunks[nck++] = SelChunk{c, first, n, q.L, q.nlist, a.hist_slot, a.pbar_off, a.idx_off};
        }
        for (int pidx = 0; pidx < nparts; ++pidx) {
          a.j0 = pidx * AVG_SPAN;
          a.j1 = std::min(q.L, (pidx + 1) * AVG_SPAN);
          post[np++] = a;
        }
        pbar += pbar_row(q.L);
      }
    }
  }
  if (pl.attn)
    for (int r = 0; r < B; ++r) {
      const int nc = pl.nchunk[r];
      if (nc == 1) continue;
      const Req& q = rq[r];
      const int rq_rows = q.verify ? rows_v : 1;
      for (int g = 0; g < Hkv; ++g) {
        PostItem m;
        std::memset(&m, 0, sizeof m);
        m.kind = POST_MERGE;
        m.hist_slot = -1;
        m.r = r;
        m.g = g;
        m.rows_q = rq_rows;
        m.L = q.L;
        m.row0 = q.row0;
        m.nchunk = nc;
        m.part_row0 = pl.part0[r] + g * (int64_t)nc * rq_rows * G;
        for (int j = 0; j < rq_rows * G; j += MERGE_ROWS) {
          m.j0 = j;
          m.j1 = std::min(rq_rows * G, j + MERGE_ROWS);
          if (pl.split && !q.verify)
            post_d[npd++] = m;
          else
            post[np++] = m;
        }
      }
    }
}

// ---- caller plan buffers -------------------------------------------------------
// A plan buffer starts with a PlanHeader.  A call that takes a buffer first
// waits until the GPU no longer reads what the previous call wrote there: that
// call's kernels stored its sequence number into each header word it armed
// (done[0], and done[1] for an overlapped step's draft launch).  The last
// reader stores it -- the post-pass or selection launch as it starts when a
// launch before it on the stream was the last to read the pinned records, the
// attention launch's last work draw when that launch is the call's only
// reader, or a one-thread release launch.  Storing from the kernels instead
// of recording an event keeps the stream free of markers: an event between
// one call's last launch and the next call's first cost a gap of about 5 us.
//
// A call marks the header `drain` before its first launch and clears it once
// every launch is queued, so a call that fails part-way leaves the buffer to
// be reused only after its device has drained.  A wait that lasts half a
// second drains the device too, so a failed device is reported instead of
// spun on.

// Waits for all work on `device`; once it has drained, every launch of the
// call that wrote a buffer on it has finished.
int32_t drain_device(int device) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  const bool switched = e == hipSuccess && cur != device;
  if (switched) e = hipSetDevice(device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (switched) (void)hipSetDevice(cur);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("plan buffer wait: ") + hipGetErrorString(e));
  return SPA_OK;
}

// A call's hold on a plan buffer: host and device addresses of its records and
// the header words its kernels store into.
struct PlanRef {
  PlanHeader* hdr = nullptr;
  char* host = nullptr;        // records (after the header)
  const char* dev = nullptr;   // the same records as the device addresses them
  uint64_t* done_dev = nullptr;  // device address of hdr->done[0]
  uint64_t seq = 0;
};

// Checks a plan buffer of `plan_bytes` for `need` bytes of records (no
// side effect on failure).
int32_t check_plan(void* h_plan, size_t plan_bytes, size_t need, char** dev_base) {
  if (!h_plan) return fail(SPA_ERR_INVALID_ARG, "h_plan is NULL");
  if ((reinterpret_cast<uintptr_t>(h_plan) & 63) != 0)
    return fail(SPA_ERR_INVALID_ARG, "h_plan must be 64-byte aligned");
  if (plan_bytes < PLAN_HEADER + need)
    return fail(SPA_ERR_PLAN_TOO_SMALL, "plan buffer of " + std::to_string(plan_bytes) +
                                            " bytes, need " + std::to_string(PLAN_HEADER + need));
  void* d = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&d, h_plan, 0);
  if (e != hipSuccess || !d) {
    (void)hipGetLastError();
    return fail(SPA_ERR_INVALID_ARG, "h_plan is not pinned host memory the device can read");
  }
  *dev_base = static_cast<char*>(d);
  return SPA_OK;
}

// Takes a checked plan buffer for a new call: waits for (or drains) the
// previous call's readers, then marks the buffer in use.
int32_t acquire_plan(void* h_plan, char* dev_base, PlanRef* out) {
  PlanHeader* h = static_cast<PlanHeader*>(h_plan);
  uint64_t prev = 0;
  if (h->magic == PLAN_MAGIC) {
    prev = h->issued;
    bool drain = h->drain != 0;
    const auto t0 = std::chrono::steady_clock::now();
    for (int b = 0; b < 2 && !drain; ++b) {
      if (!((h->need >> b) & 1u)) continue;
      while (__atomic_load_n(&h->done[b], __ATOMIC_ACQUIRE) < prev) {
        std::this_thread::yield();
        if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(500)) {
          drain = true;
          break;
        }
      }
    }
    if (drain) {
      const int32_t rc = drain_device(h->device);
      if (rc) return rc;
    }
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SPA_ERR_HIP, "no current device");
  h->need = 0;
  h->drain = 1;  // until every launch of this call is queued
  h->device = dev;
  h->issued = prev + 1;
  __atomic_store_n(&h->magic, PLAN_MAGIC, __ATOMIC_RELEASE);
  out->hdr = h;
  out->host = static_cast<char*>(h_plan) + PLAN_HEADER;
  out->dev = dev_base + PLAN_HEADER;
  out->done_dev = reinterpret_cast<uint64_t*>(dev_base + offsetof(PlanHeader, done));
  out->seq = prev + 1;
  return SPA_OK;
}

// Every launch of the call is queued: a later call waits for the armed words.
void arm_plan(PlanRef& pr, uint32_t need) {
  pr.hdr->need = need;
  __atomic_store_n(&pr.hdr->drain, 0, __ATOMIC_RELEASE);
}

// Records an optional timing event on a stream.
hipError_t mark(hipEvent_t ev, hipStream_t st) { return ev ? hipEventRecord(ev, st) : hipSuccess; }

struct Buffers {
  const int32_t* page_table = nullptr;
  const void* q = nullptr;
  const void* k_pool = nullptr;
  const void* v_pool = nullptr;
  const int32_t* idx_in = nullptr;
  int32_t* idx_out = nullptr;
  void* o = nullptr;
  float* lse = nullptr;
  float* logits = nullptr;
};

int32_t run(const Shape& s, const std::vector<Req>& rq, const Plan& pl, const Buffers& b,
            int avg_begin, int avg_count, void* d_ws, size_t ws_bytes, void* h_plan,
            size_t plan_bytes, const Opts& o, hipStream_t st) {
  if (ws_bytes < pl.total)
    return fail(SPA_ERR_WORKSPACE_TOO_SMALL,
                "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(pl.total));
  if (!d_ws) return fail(SPA_ERR_INVALID_ARG, "d_ws is NULL");
  if ((reinterpret_cast<uintptr_t>(d_ws) & 255) != 0)
    return fail(SPA_ERR_INVALID_ARG, "d_ws must be 256-byte aligned");
  const int n_post = pl.n_avg + pl.n_merge;
  if (pl.n_items == 0 && pl.n_items_d == 0 && n_post == 0 && pl.n_sel == 0) return SPA_OK;
  char* dev_base = nullptr;
  int32_t rc = check_plan(h_plan, plan_bytes, pl.h_bytes, &dev_base);
  if (rc) return rc;
  PlanRef pr;
  rc = acquire_plan(h_plan, dev_base, &pr);
  if (rc) return rc;
  plan_write(s, rq, pl, pr.host);
  const char* plan = pr.dev;
  char* ws = static_cast<char*>(d_ws);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(ws);  // [0]: attention on `st`, [1]: draft launch
  void* part_o = ws + pl.off_part_o;
  float* part_ml = reinterpret_cast<float*>(ws + pl.off_part_ml);
  hipError_t e = hipSuccess;
  if (pl.n_items > 0 || pl.n_items_d > 0) {
    AttnParams p;
    p.items = reinterpret_cast<const Item*>(plan + pl.h_items);
    p.q = b.q;
    p.k_pool = b.k_pool;
    p.v_pool = b.v_pool;
    p.page_table = b.page_table;
    p.pt_stride = s.stride;
    p.num_slots = s.num_slots;
    p.idx_in = b.idx_in;
    p.o = b.o;
    p.lse = b.lse;
    p.logits = b.logits;
    p.part_o = part_o;
    p.part_ml = part_ml;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.k = s.k;
    p.sm_scale = s.scale;
    p.ticket = tickets;
    // the launch on `st` moves the records of the launches that follow it
    p.plan_src = reinterpret_cast<const uint4*>(plan + pl.h_post);
    p.plan_dst = reinterpret_cast<uint4*>(ws + pl.off_plan);
    p.plan_n16 = pl.n_items > 0 ? static_cast<int32_t>((pl.h_bytes - pl.h_post) / 16) : 0;
    // ... and clears the score histograms the post-pass adds to
    p.zero_dst = reinterpret_cast<uint4*>(ws + pl.off_hist);
    p.zero_n16 = pl.n_items > 0 ? static_cast<int32_t>(pl.hist_zero_bytes / 16) : 0;
    // a call that is this one launch reports its plan free from the launch
    const bool attn_only = pl.n_items > 0 && n_post == 0 && pl.n_sel == 0 && !pl.split;
    p.done = attn_only ? pr.done_dev : nullptr;
    p.done_val = pr.seq;
    if (pl.split) {
      // the fork point: everything already on `st`, but not the verify attention
      e = hipEventRecord(o.fork, st);
      if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("fork: ") + hipGetErrorString(e));
    }
    // verify (or all) attention first, so that its long items reach the CUs
    // before the draft launch's
    if (pl.n_items > 0) {
      e = mark(o.timing[0], st);
      if (e == hipSuccess) e = launch_attn(p, s.dtype, s.d, pl.n_items, pl.nthr, pl.smem, false, st);
      if (e == hipSuccess) e = mark(o.timing[1], st);
      if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(e));
    }
    if (pl.split) {
      e = hipStreamWaitEvent(o.side, o.fork, 0);
      if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("fork wait: ") + hipGetErrorString(e));
      AttnParams pd = p;
      pd.items = reinterpret_cast<const Item*>(plan + pl.h_items_d);
      pd.ticket = tickets + 1;
      pd.plan_n16 = 0;
      pd.zero_n16 = 0;
      pd.done = pr.done_dev + 1;  // its last work draw releases its records
      e = mark(o.timing[6], o.side);
      if (e == hipSuccess)
        e = launch_attn(pd, s.dtype, s.d, pl.n_items_d, pl.nthr, pl.smem, true, o.side);
      if (e == hipSuccess) e = mark(o.timing[7], o.side);
      if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("draft attention launch: ") + hipGetErrorString(e));
      e = hipEventRecord(o.join, o.side);
      if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("join record: ") + hipGetErrorString(e));
    }
  }
  // records of the launches below: the workspace copy, made by the attention
  // launch on `st` or (without one) by the post-pass for the selection launch
  const bool attn_st = pl.n_items > 0;
  auto ws_rec = [&](size_t h_off) {
    return reinterpret_cast<const PostItem*>(ws + pl.off_plan + (h_off - pl.h_post));
  };
  // selected rows' score histograms: cleared by the attention launch on `st`
  uint32_t* hist = (attn_st && pl.n_hist > 0) ? reinterpret_cast<uint32_t*>(ws + pl.off_hist) : nullptr;
  if (n_post > 0) {
    PostParams pp;
    pp.items = attn_st ? ws_rec(pl.h_post) : reinterpret_cast<const PostItem*>(plan + pl.h_post);
    pp.part_o = part_o;
    pp.part_ml = part_ml;
    pp.o = b.o;
    pp.lse = b.lse;
    pp.logits = b.logits;
    pp.pbar = reinterpret_cast<float*>(ws + pl.off_pbar);
    pp.Hq = s.Hq;
    pp.G = s.G;
    pp.avg_row_begin = avg_begin;
    pp.avg_row_count = avg_count;
    // logits that the Infinity Cache can still hold when the post-pass reads
    // them back: plain loads, which hit there; otherwise the streaming hint
    pp.logits_cached = attn_st && pl.avg_logit_bytes <= LOGITS_CACHED_BYTES;
    // the attention launch before it read the pinned records last
    pp.done = attn_st ? pr.done_dev : nullptr;
    pp.done_val = pr.seq;
    pp.hist = hist;
    pp.plan_src = reinterpret_cast<const uint4*>(plan + pl.h_sel);
    pp.plan_dst = reinterpret_cast<uint4*>(ws + pl.off_plan + (pl.h_sel - pl.h_post));
    pp.plan_n16 = attn_st ? 0 : static_cast<int32_t>((pl.h_bytes - pl.h_sel) / 16);
    e = mark(o.timing[2], st);
    if (e == hipSuccess)
      e = launch_post(pp, s.dtype, s.d, n_post,
                      post_smem_bytes(pl.n_avg ? avg_count * s.G : 0, pl.max_nchunk, hist != nullptr), st);
    if (e == hipSuccess) e = mark(o.timing[3], st);
    if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("post-pass launch: ") + hipGetErrorString(e));
  }
  if (pl.n_sel > 0) {
    SelectParams sp;
    sp.items = ws_rec(pl.h_sel);
    sp.pbar = reinterpret_cast<const float*>(ws + pl.off_pbar);
    sp.idx_out = b.idx_out;
    sp.hist = hist;
    // long rows in chunks (their histograms are there), every other row by
    // one workgroup, through the LDS position bitmap when it is long
    const bool chunked = hist != nullptr && pl.n_chunks > 0;
    sp.bm_bits = select_bitmap_bits(chunked ? pl.max_row_sel_len : pl.max_sel_len);
    sp.n_sel = pl.n_sel;
    sp.n_chunks = chunked ? pl.n_chunks : 0;
    sp.chunks = reinterpret_cast<const SelChunk*>(ws + pl.off_plan + (pl.h_chunks - pl.h_post));
    sp.row_info = reinterpret_cast<uint32_t*>(ws + pl.off_row_info);
    sp.cnt_above = reinterpret_cast<uint32_t*>(ws + pl.off_cnt_above);
    sp.cnt_bin = reinterpret_cast<uint32_t*>(ws + pl.off_cnt_bin);
    sp.cand_key = reinterpret_cast<uint32_t*>(ws + pl.off_cand_key);
    sp.cand_pos = reinterpret_cast<int32_t*>(ws + pl.off_cand_pos);
    // without an attention launch, the post-pass before it read the pinned records last
    sp.done = attn_st ? nullptr : pr.done_dev;
    sp.done_val = pr.seq;
    e = mark(o.timing[4], st);
    // the per-row launch only when some row is not chunked
    const bool rows = !chunked || pl.n_chunked_rows < pl.n_sel;
    if (e == hipSuccess) e = launch_select_count(sp, st);
    if (e == hipSuccess && rows) e = launch_select(sp, pl.n_sel, st);
    if (e == hipSuccess) e = launch_select_chunks(sp, st);
    if (e == hipSuccess) e = mark(o.timing[5], st);
    if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("selection launch: ") + hipGetErrorString(e));
  }
  if (pl.split) {
    e = hipStreamWaitEvent(st, o.join, 0);
    if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("join: ") + hipGetErrorString(e));
    if (pl.n_merge_d > 0) {  // merges of drafts split into several chunks
      PostParams pp;
      pp.items = ws_rec(pl.h_post_d);
      pp.part_o = part_o;
      pp.part_ml = part_ml;
      pp.o = b.o;
      pp.lse = b.lse;
      pp.logits = b.logits;
      pp.pbar = nullptr;
      pp.Hq = s.Hq;
      pp.G = s.G;
      pp.avg_row_begin = avg_begin;
      pp.avg_row_count = avg_count;
      pp.logits_cached = false;
      pp.done = nullptr;
      pp.done_val = 0;
      pp.hist = nullptr;
      pp.plan_src = nullptr;
      pp.plan_dst = nullptr;
      pp.plan_n16 = 0;
      e = launch_post(pp, s.dtype, s.d, pl.n_merge_d, post_smem_bytes(0, pl.max_nchunk, false), st);
      if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("draft merge launch: ") + hipGetErrorString(e));
    }
  }
  arm_plan(pr, pl.split ? 3u : 1u);
  return SPA_OK;
}

int32_t check_avg_rows(int k, int G, int begin, int count) {
  if (begin < 0 || count < 1 || begin + count > k + 1)
    return fail(SPA_ERR_INVALID_ARG, "averaged rows must lie in [0, k]");
  if (count * G > MAX_AVG_TERMS)
    return fail(SPA_ERR_UNSUPPORTED, "averaged rows times GQA group above 512");
  return SPA_OK;
}

// Shared request checks.  verify: L >= k+1 and K in [1, L]; draft: list >= 1.
int32_t collect(const Shape& s, int B, const uint8_t* is_verify, const int32_t* seq_lens,
                const int32_t* q_indptr, const int32_t* counts, const int64_t* idx_off,
                const int64_t* logits_off, bool need_logits, bool need_idx,
                std::vector<Req>* out) {
  out->resize(B);
  int32_t row = q_indptr ? q_indptr[0] : 0;
  if (row < 0) return fail(SPA_ERR_INVALID_ARG, "q_indptr[0] is negative");
  for (int r = 0; r < B; ++r) {
    Req& q = (*out)[r];
    q.verify = is_verify ? is_verify[r] != 0 : false;
    q.L = seq_lens[r];
    if (q.L < 1) return fail(SPA_ERR_INVALID_ARG, "seq_lens[" + std::to_string(r) + "] < 1");
    if (q.L > s.stride)
      return fail(SPA_ERR_INVALID_ARG, "seq_lens[" + std::to_string(r) + "] exceeds page_table_stride");
    if (q.verify && q.L < s.k + 1)
      return fail(SPA_ERR_INVALID_ARG, "verify request " + std::to_string(r) + " shorter than k+1");
    const int rows = q.verify ? s.k + 1 : 1;
    if (q_indptr) {
      if (q_indptr[r + 1] - q_indptr[r] != rows)
        return fail(SPA_ERR_INVALID_ARG, "q_indptr row count of request " + std::to_string(r) +
                                             " must be " + std::to_string(rows));
      q.row0 = q_indptr[r];
    } else {
      q.row0 = row;
      row += rows;
    }
    if (counts) {
      q.nlist = counts[r];
      if (q.verify && (q.nlist < 1 || q.nlist > q.L))
        return fail(SPA_ERR_INVALID_ARG, "top-K count of request " + std::to_string(r) + " outside [1, L]");
      if (!q.verify && q.nlist < 1)
        return fail(SPA_ERR_INVALID_ARG, "index list of request " + std::to_string(r) + " is empty");
    }
    q.idx_off = idx_off ? idx_off[r] : 0;
    q.logits_off = (logits_off && q.verify) ? logits_off[r] : 0;
  }
  if (need_idx) {
    std::vector<std::pair<int64_t, int64_t>> seg;
    for (auto& q : *out) seg.push_back({q.idx_off, (int64_t)s.Hkv * q.nlist});
    int32_t rc = check_segments(seg, "idx offsets");
    if (rc) return rc;
  }
  if (need_logits) {
    std::vector<std::pair<int64_t, int64_t>> seg;
    for (auto& q : *out)
      if (q.verify) seg.push_back({q.logits_off, (int64_t)(s.k + 1) * s.Hq * q.L});
    int32_t rc = check_segments(seg, "logits offsets");
    if (rc) return rc;
  }
  return SPA_OK;
}

// Address ranges [begin, end) of int32 list segments; two output ranges, or an
// output and an input range, must not share an element.
struct Range {
  uintptr_t begin, end;
  bool out;
};
int32_t check_no_overlap(std::vector<Range> v) {
  std::sort(v.begin(), v.end(),
            [](const Range& a, const Range& b) { return a.begin < b.begin; });
  // sweep: the furthest end so far of output ranges and of input ranges
  uintptr_t out_end = 0, in_end = 0;
  for (const Range& x : v) {
    if (x.begin == x.end) continue;
    if (x.begin < out_end || (x.out && x.begin < in_end))
      return fail(SPA_ERR_INVALID_ARG, "output lists overlap each other or a stored list");
    (x.out ? out_end : in_end) = std::max(x.out ? out_end : in_end, x.end);
  }
  return SPA_OK;
}

}  // namespace

extern "C" {

int32_t spa_abi_version(void) { return SPA_ABI_VERSION; }

const char* spa_last_error(void) { return g_err.c_str(); }

namespace {
// The unified step's plan for a batch: it needs the most workspace and plan
// bytes of the four attention entry points.
int32_t size_plan(const spa_layout* layout, int32_t B, int32_t spec_k, const uint8_t* h_is_verify,
                  const int32_t* h_seq_lens, const int32_t* h_idx_count, const spa_options* opts,
                  Plan* pl) {
  Shape s;
  int32_t rc = check_layout(layout, &s);
  if (rc) return rc;
  Opts o;
  rc = check_opts(opts, &o);
  if (rc) return rc;
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (B == 0) return SPA_OK;
  if (!h_seq_lens) return fail(SPA_ERR_INVALID_ARG, "h_seq_lens is NULL");
  bool any_v = false;
  for (int r = 0; r < B && h_is_verify; ++r) any_v |= h_is_verify[r] != 0;
  if (any_v && spec_k < 1) return fail(SPA_ERR_INVALID_ARG, "spec_k < 1");
  s.k = std::max(spec_k, 0);
  std::vector<int32_t> counts(B);
  for (int r = 0; r < B; ++r) counts[r] = h_idx_count ? h_idx_count[r] : 1;
  std::vector<Req> rq;
  rc = collect(s, B, h_is_verify, h_seq_lens, nullptr, counts.data(), nullptr, nullptr, false,
               false, &rq);
  if (rc) return rc;
  // sizes do not depend on the overlap streams being given
  o.side = reinterpret_cast<hipStream_t>(1);
  o.fork = o.join = reinterpret_cast<hipEvent_t>(1);
  return plan_size(s, rq, true, true, o, pl);
}
}  // namespace

size_t spa_workspace_bytes(const spa_layout* layout, int32_t B, int32_t spec_k,
                           const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                           const int32_t* h_idx_count, const spa_options* opts) {
  Plan pl;
  if (size_plan(layout, B, spec_k, h_is_verify, h_seq_lens, h_idx_count, opts, &pl)) return 0;
  return B == 0 ? 0 : pl.total;
}

size_t spa_plan_bytes(const spa_layout* layout, int32_t B, int32_t spec_k,
                      const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                      const int32_t* h_idx_count, const spa_options* opts) {
  Plan pl;
  if (size_plan(layout, B, spec_k, h_is_verify, h_seq_lens, h_idx_count, opts, &pl)) return 0;
  return B == 0 ? 0 : PLAN_HEADER + pl.h_bytes;
}

int32_t spa_verify_attn(const spa_layout* layout, int32_t B, int32_t spec_k,
                        const int32_t* h_seq_lens, const int32_t* d_page_table, const void* d_q,
                        const void* d_k_pool, const void* d_v_pool, void* d_o, float* d_lse,
                        float* d_logits, const int64_t* h_logits_off, void* d_ws,
                        size_t ws_bytes, void* h_plan, size_t plan_bytes,
                        const spa_options* opts, void* stream) {
  Shape s;
  int32_t rc = check_layout(layout, &s);
  if (rc) return rc;
  Opts o;
  rc = check_opts(opts, &o);
  if (rc) return rc;
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (spec_k < 1) return fail(SPA_ERR_INVALID_ARG, "spec_k < 1");
  if (B == 0) return SPA_OK;
  if (!h_seq_lens || !d_page_table || !d_q || !d_k_pool || !d_v_pool || !d_o || !d_lse ||
      !d_logits || !h_logits_off)
    return fail(SPA_ERR_INVALID_ARG, "a required pointer is NULL");
  s.k = spec_k;
  std::vector<uint8_t> ver(B, 1);
  std::vector<Req> rq;
  rc = collect(s, B, ver.data(), h_seq_lens, nullptr, nullptr, nullptr, h_logits_off, true, false,
               &rq);
  if (rc) return rc;
  rc = apply_pt_rows(o, &rq);
  if (rc) return rc;
  Plan pl;
  rc = plan_size(s, rq, true, false, o, &pl);
  if (rc) return rc;
  Buffers b;
  b.page_table = d_page_table;
  b.q = d_q;
  b.k_pool = d_k_pool;
  b.v_pool = d_v_pool;
  b.o = d_o;
  b.lse = d_lse;
  b.logits = d_logits;
  return run(s, rq, pl, b, 1, spec_k, d_ws, ws_bytes, h_plan, plan_bytes, o,
             static_cast<hipStream_t>(stream));
}

int32_t spa_pillar_topk(int32_t B, int32_t spec_k, int32_t num_qo_heads, int32_t num_kv_heads,
                        int32_t avg_row_begin, int32_t avg_row_count, const int32_t* h_seq_lens,
                        const int32_t* h_topk, const float* d_logits,
                        const int64_t* h_logits_off, const float* d_lse, int32_t* d_idx,
                        const int64_t* h_idx_off, void* d_ws, size_t ws_bytes, void* h_plan,
                        size_t plan_bytes, const spa_options* opts, void* stream) {
  if (num_qo_heads <= 0 || num_kv_heads <= 0 || num_qo_heads % num_kv_heads != 0)
    return fail(SPA_ERR_INVALID_ARG, "head counts must be positive with H_q % H_kv == 0");
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (spec_k < 1) return fail(SPA_ERR_INVALID_ARG, "spec_k < 1");
  Opts o;
  int32_t rc = check_opts(opts, &o);
  if (rc) return rc;
  Shape s;
  s.Hq = num_qo_heads;
  s.Hkv = num_kv_heads;
  s.G = num_qo_heads / num_kv_heads;
  s.d = 128;
  s.k = spec_k;
  s.stride = 0x7fffffff;
  rc = check_avg_rows(spec_k, s.G, avg_row_begin, avg_row_count);
  if (rc) return rc;
  if (B == 0) return SPA_OK;
  if (!h_seq_lens || !h_topk || !d_logits || !h_logits_off || !d_lse || !d_idx || !h_idx_off)
    return fail(SPA_ERR_INVALID_ARG, "a required pointer is NULL");
  std::vector<uint8_t> ver(B, 1);
  std::vector<Req> rq;
  rc = collect(s, B, ver.data(), h_seq_lens, nullptr, h_topk, h_idx_off, h_logits_off, true, true,
               &rq);
  if (rc) return rc;
  Plan pl;
  rc = plan_size(s, rq, false, true, o, &pl);
  if (rc) return rc;
  Buffers b;
  b.logits = const_cast<float*>(d_logits);
  b.lse = const_cast<float*>(d_lse);
  b.idx_out = d_idx;
  return run(s, rq, pl, b, avg_row_begin, avg_row_count, d_ws, ws_bytes, h_plan, plan_bytes, o,
             static_cast<hipStream_t>(stream));
}

int32_t spa_draft_attn(const spa_layout* layout, int32_t B, const int32_t* h_seq_lens,
                       const int32_t* d_page_table, const int32_t* h_idx_count,
                       const int64_t* h_idx_off, const int32_t* d_idx, const void* d_q,
                       const void* d_k_pool, const void* d_v_pool, void* d_o, float* d_lse,
                       void* d_ws, size_t ws_bytes, void* h_plan, size_t plan_bytes,
                       const spa_options* opts, void* stream) {
  Shape s;
  int32_t rc = check_layout(layout, &s);
  if (rc) return rc;
  Opts o;
  rc = check_opts(opts, &o);
  if (rc) return rc;
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (B == 0) return SPA_OK;
  if (!h_seq_lens || !d_page_table || !h_idx_count || !h_idx_off || !d_idx || !d_q ||
      !d_k_pool || !d_v_pool || !d_o || !d_lse)
    return fail(SPA_ERR_INVALID_ARG, "a required pointer is NULL");
  s.k = 0;
  std::vector<Req> rq;
  rc = collect(s, B, nullptr, h_seq_lens, nullptr, h_idx_count, h_idx_off, nullptr, false, true,
               &rq);
  if (rc) return rc;
  rc = apply_pt_rows(o, &rq);
  if (rc) return rc;
  Plan pl;
  rc = plan_size(s, rq, true, false, o, &pl);
  if (rc) return rc;
  Buffers b;
  b.page_table = d_page_table;
  b.q = d_q;
  b.k_pool = d_k_pool;
  b.v_pool = d_v_pool;
  b.idx_in = d_idx;
  b.o = d_o;
  b.lse = d_lse;
  return run(s, rq, pl, b, 0, 1, d_ws, ws_bytes, h_plan, plan_bytes, o,
             static_cast<hipStream_t>(stream));
}

int32_t spa_unified_step(const spa_layout* layout, int32_t B, int32_t spec_k,
                         const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                         const int32_t* h_q_indptr, const int32_t* d_page_table,
                         const void* d_q, const void* d_k_pool, const void* d_v_pool,
                         const int32_t* h_idx_count, const int64_t* h_idx_off, int32_t* d_idx,
                         void* d_o, float* d_lse, float* d_logits, const int64_t* h_logits_off,
                         int32_t avg_row_begin, int32_t avg_row_count, void* d_ws,
                         size_t ws_bytes, void* h_plan, size_t plan_bytes,
                         const spa_options* opts, void* stream) {
  Shape s;
  int32_t rc = check_layout(layout, &s);
  if (rc) return rc;
  Opts o;
  rc = check_opts(opts, &o);
  if (rc) return rc;
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (spec_k < 1) return fail(SPA_ERR_INVALID_ARG, "spec_k < 1");
  rc = check_avg_rows(spec_k, s.G, avg_row_begin, avg_row_count);
  if (rc) return rc;
  if (B == 0) return SPA_OK;
  if (!h_is_verify || !h_seq_lens || !h_q_indptr || !d_page_table || !d_q || !d_k_pool ||
      !d_v_pool || !h_idx_count || !h_idx_off || !d_idx || !d_o || !d_lse)
    return fail(SPA_ERR_INVALID_ARG, "a required pointer is NULL");
  bool any_v = false;
  for (int r = 0; r < B; ++r) any_v |= h_is_verify[r] != 0;
  if (any_v && (!d_logits || !h_logits_off))
    return fail(SPA_ERR_INVALID_ARG, "verify requests need d_logits and h_logits_off");
  s.k = spec_k;
  std::vector<Req> rq;
  rc = collect(s, B, h_is_verify, h_seq_lens, h_q_indptr, h_idx_count, h_idx_off, h_logits_off,
               any_v, true, &rq);
  if (rc) return rc;
  rc = apply_pt_rows(o, &rq);
  if (rc) return rc;
  Plan pl;
  rc = plan_size(s, rq, true, true, o, &pl);
  if (rc) return rc;
  Buffers b;
  b.page_table = d_page_table;
  b.q = d_q;
  b.k_pool = d_k_pool;
  b.v_pool = d_v_pool;
  b.idx_in = d_idx;
  b.idx_out = d_idx;
  b.o = d_o;
  b.lse = d_lse;
  b.logits = d_logits;
  return run(s, rq, pl, b, avg_row_begin, avg_row_count, d_ws, ws_bytes, h_plan, plan_bytes, o,
             static_cast<hipStream_t>(stream));
}

// ---- the entry point that allocates nothing ---------------------------------
// spa_unified_step_static runs the unified step with its workspace in this
// file-scope device array instead of a caller buffer.  Each GPU holds its own
// copy until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns on that device (the array's name is a host-side
// stand-in, not a device address).  Its first bytes are the attention work
// counters: zero at load, and every call leaves them zero.
static __device__ __align__(256) char scratch[SPA_STATIC_WORKSPACE_BYTES];
}  // extern "C"

namespace {
// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int32_t scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("get device: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(SPA_ERR_HIP, std::string("static workspace address: ") + hipGetErrorString(e));
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return SPA_OK;
}
}  // namespace

extern "C" {

int32_t spa_unified_step_static(const spa_layout* layout, int32_t B, int32_t spec_k,
                                const uint8_t* h_is_verify, const int32_t* h_seq_lens,
                                const int32_t* h_q_indptr, const int32_t* d_page_table,
                                const void* d_q, const void* d_k_pool, const void* d_v_pool,
                                const int32_t* h_idx_count, const int64_t* h_idx_off,
                                int32_t* d_idx, void* d_o, float* d_lse, float* d_logits,
                                const int64_t* h_logits_off, int32_t avg_row_begin,
                                int32_t avg_row_count, void* h_plan, size_t plan_bytes,
                                const spa_options* opts, void* stream) {
  // the arguments are checked and the batch sized before the array is used
  if (B > 0) {
    const size_t need = spa_workspace_bytes(layout, B, spec_k, h_is_verify, h_seq_lens,
                                            h_idx_count, opts);
    if (need == 0) {
      // invalid sizes: the full call reports the precise reason
      return spa_unified_step(layout, B, spec_k, h_is_verify, h_seq_lens, h_q_indptr,
                              d_page_table, d_q, d_k_pool, d_v_pool, h_idx_count, h_idx_off,
                              d_idx, d_o, d_lse, d_logits, h_logits_off, avg_row_begin,
                              avg_row_count, nullptr, 0, h_plan, plan_bytes, opts, stream);
    }
    if (need > SPA_STATIC_WORKSPACE_BYTES)
      return fail(SPA_ERR_UNSUPPORTED,
                  "batch needs a workspace of " + std::to_string(need) +
                      " bytes, above the static workspace's " +
                      std::to_string((size_t)SPA_STATIC_WORKSPACE_BYTES) +
                      "; use spa_unified_step with a caller workspace");
  }
  void* ws = nullptr;
  if (B > 0) {
    const int32_t rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return spa_unified_step(layout, B, spec_k, h_is_verify, h_seq_lens, h_q_indptr, d_page_table,
                          d_q, d_k_pool, d_v_pool, h_idx_count, h_idx_off, d_idx, d_o, d_lse,
                          d_logits, h_logits_off, avg_row_begin, avg_row_count, ws,
                          SPA_STATIC_WORKSPACE_BYTES, h_plan, plan_bytes, opts, stream);
}

size_t spa_recall_plan_bytes(int32_t B) {
  return B < 0 ? 0 : PLAN_HEADER + (size_t)B * sizeof(RecallReq);
}

size_t spa_list_quality_plan_bytes(int32_t B) {
  return B < 0 ? 0 : PLAN_HEADER + (size_t)B * sizeof(QualityReq);
}

int32_t spa_recall_index(int32_t B, int32_t num_kv_heads, const int32_t* h_seq_lens,
                         int32_t n_sink, int32_t n_recent, const int32_t* h_in_count,
                         const int64_t* h_in_off, const int32_t* d_idx_in,
                         const int32_t* h_out_count, const int64_t* h_out_off, int32_t* d_idx_out,
                         void* h_plan, size_t plan_bytes, void* stream) {
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (num_kv_heads <= 0) return fail(SPA_ERR_INVALID_ARG, "num_kv_heads must be positive");
  if (n_sink < 0 || n_recent < 0) return fail(SPA_ERR_INVALID_ARG, "n_sink and n_recent must be >= 0");
  if (B == 0) return SPA_OK;
  if (!h_seq_lens || !h_in_count || !h_in_off || !h_out_count || !h_out_off || !d_idx_out)
    return fail(SPA_ERR_INVALID_ARG, "a required pointer is NULL");
  std::vector<Range> ranges;
  ranges.reserve(2 * (size_t)B);
  int max_len = 1;
  bool any_in = false;
  for (int r = 0; r < B; ++r) {
    const int64_t L = h_seq_lens[r], n_in = h_in_count[r], n_out = h_out_count[r];
    if (L < 1) return fail(SPA_ERR_INVALID_ARG, "request " + std::to_string(r) + ": L < 1");
    if (L > MAX_RECALL_LEN)
      return fail(SPA_ERR_UNSUPPORTED, "request " + std::to_string(r) + ": L above 1048576");
    if (n_in < 0) return fail(SPA_ERR_INVALID_ARG, "request " + std::to_string(r) + ": stored count < 0");
    const int64_t s_end = std::min<int64_t>(n_sink, L);
    const int64_t r_begin = std::max<int64_t>(s_end, L - std::min<int64_t>(n_recent, L));
    const int64_t bound = std::min<int64_t>(L, s_end + (L - r_begin) + n_in);
    if (n_out < std::max<int64_t>(bound, 1))
      return fail(SPA_ERR_INVALID_ARG, "request " + std::to_string(r) + ": output length " +
                                           std::to_string(n_out) + " below " +
                                           std::to_string(std::max<int64_t>(bound, 1)));
    if (h_in_off[r] < 0 || h_out_off[r] < 0)
      return fail(SPA_ERR_INVALID_ARG, "request " + std::to_string(r) + ": negative offset");
    max_len = std::max<int>(max_len, (int)L);
    if (n_in > 0) {
      any_in = true;
      const uintptr_t a = reinterpret_cast<uintptr_t>(d_idx_in) + (uintptr_t)h_in_off[r] * 4;
      ranges.push_back(Range{a, a + (uintptr_t)(n_in * num_kv_heads) * 4, false});
    }
    const uintptr_t a = reinterpret_cast<uintptr_t>(d_idx_out) + (uintptr_t)h_out_off[r] * 4;
    ranges.push_back(Range{a, a + (uintptr_t)(n_out * num_kv_heads) * 4, true});
  }
  if (any_in && !d_idx_in) return fail(SPA_ERR_INVALID_ARG, "d_idx_in is NULL");
  int32_t rc = check_no_overlap(std::move(ranges));
  if (rc) return rc;
  if ((int64_t)B * num_kv_heads > 0x7fffffff)
    return fail(SPA_ERR_UNSUPPORTED, "more than 2^31 - 1 (request, KV head) pairs");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* dev_base = nullptr;
  rc = check_plan(h_plan, plan_bytes, (size_t)B * sizeof(RecallReq), &dev_base);
  if (rc) return rc;
  PlanRef pr;
  rc = acquire_plan(h_plan, dev_base, &pr);
  if (rc) return rc;
  RecallReq* rec = reinterpret_cast<RecallReq*>(pr.host);
  for (int r = 0; r < B; ++r) {
    rec[r].L = h_seq_lens[r];
    rec[r].in_count = h_in_count[r];
    rec[r].out_count = h_out_count[r];
    rec[r].pad_ = 0;
    rec[r].in_off = h_in_off[r];
    rec[r].out_off = h_out_off[r];
  }
  RecallParams rp;
  rp.reqs = reinterpret_cast<const RecallReq*>(pr.dev);
  rp.idx_in = d_idx_in;
  rp.idx_out = d_idx_out;
  rp.Hkv = num_kv_heads;
  rp.n_sink = n_sink;
  rp.n_recent = n_recent;
  hipError_t e = launch_recall(rp, B * num_kv_heads, recall_smem_bytes(max_len), st);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("recall launch: ") + hipGetErrorString(e));
  e = launch_release(pr.done_dev, pr.seq, st);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("release launch: ") + hipGetErrorString(e));
  arm_plan(pr, 1u);
  return SPA_OK;
}

size_t spa_list_quality_workspace_bytes(int32_t B, int32_t num_qo_heads,
                                        const int32_t* h_seq_lens) {
  if (B <= 0 || num_qo_heads <= 0 || !h_seq_lens) return 0;
  size_t total = 0;
  for (int r = 0; r < B; ++r)
    total += (size_t)num_qo_heads * (size_t)((std::max(h_seq_lens[r], 0) + 3) & ~3) * 4;
  return total;
}

int32_t spa_list_quality(int32_t B, int32_t spec_k, int32_t num_qo_heads, int32_t num_kv_heads,
                         int32_t row, int32_t top_t, const int32_t* h_seq_lens,
                         const float* d_logits, const int64_t* h_logits_off, const float* d_lse,
                         const int32_t* h_list_count, const int64_t* h_list_off,
                         const int32_t* d_list, int32_t* d_top, float* d_coverage,
                         float* d_recall, void* d_ws, size_t ws_bytes, void* h_plan,
                         size_t plan_bytes, void* stream) {
  if (B < 0) return fail(SPA_ERR_INVALID_ARG, "B < 0");
  if (num_qo_heads <= 0 || num_kv_heads <= 0 || num_qo_heads % num_kv_heads != 0)
    return fail(SPA_ERR_INVALID_ARG, "head counts must be positive with H_q % H_kv == 0");
  if (spec_k < 1) return fail(SPA_ERR_INVALID_ARG, "spec_k < 1");
  if (row < 0 || row > spec_k) return fail(SPA_ERR_INVALID_ARG, "row must lie in [0, spec_k]");
  if (top_t < 1) return fail(SPA_ERR_INVALID_ARG, "top_t < 1");
  if (B == 0) return SPA_OK;
  if (!h_seq_lens || !d_logits || !h_logits_off || !d_lse || !h_list_count || !h_list_off ||
      !d_top || !d_coverage || !d_recall)
    return fail(SPA_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((int64_t)B * num_qo_heads > 0x7fffffff)
    return fail(SPA_ERR_UNSUPPORTED, "more than 2^31 - 1 (request, query head) pairs");
  int max_len = 1;
  bool any_list = false;
  std::vector<std::pair<int64_t, int64_t>> seg;
  for (int r = 0; r < B; ++r) {
    const int32_t L = h_seq_lens[r];
    const std::string who = "request " + std::to_string(r);
    if (L < spec_k + 1) return fail(SPA_ERR_INVALID_ARG, who + ": L < spec_k + 1");
    if (L > MAX_RECALL_LEN) return fail(SPA_ERR_UNSUPPORTED, who + ": L above 1048576");
    if (top_t > L) return fail(SPA_ERR_INVALID_ARG, who + ": top_t > L");
    if (h_list_count[r] < 0) return fail(SPA_ERR_INVALID_ARG, who + ": list count < 0");
    if (h_logits_off[r] < 0 || h_list_off[r] < 0) return fail(SPA_ERR_INVALID_ARG, who + ": negative offset");
    any_list |= h_list_count[r] > 0;
    max_len = std::max<int>(max_len, L);
    seg.push_back({h_logits_off[r], (int64_t)(spec_k + 1) * num_qo_heads * L});
  }
  if (any_list && !d_list) return fail(SPA_ERR_INVALID_ARG, "d_list is NULL");
  int32_t rc = check_segments(std::move(seg), "logits offsets");
  if (rc) return rc;
  const size_t need = spa_list_quality_workspace_bytes(B, num_qo_heads, h_seq_lens);
  if (ws_bytes < need)
    return fail(SPA_ERR_WORKSPACE_TOO_SMALL,
                "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(need));
  if (!d_ws) return fail(SPA_ERR_INVALID_ARG, "d_ws is NULL");
  if ((reinterpret_cast<uintptr_t>(d_ws) & 15) != 0)
    return fail(SPA_ERR_INVALID_ARG, "d_ws must be 16-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* dev_base = nullptr;
  rc = check_plan(h_plan, plan_bytes, (size_t)B * sizeof(QualityReq), &dev_base);
  if (rc) return rc;
  PlanRef pr;
  rc = acquire_plan(h_plan, dev_base, &pr);
  if (rc) return rc;
  QualityReq* rec = reinterpret_cast<QualityReq*>(pr.host);
  int64_t p_off = 0;
  for (int r = 0; r < B; ++r) {
    const int32_t L = h_seq_lens[r];
    rec[r].L = L;
    rec[r].n = h_list_count[r];
    rec[r].logits_off = h_logits_off[r];
    rec[r].list_off = h_list_off[r];
    rec[r].p_off = p_off;
    rec[r].lse_row = r * (spec_k + 1) + row;
    rec[r].pad_ = 0;
    p_off += (int64_t)num_qo_heads * ((L + 3) & ~3);
  }
  QualityParams qp;
  qp.reqs = reinterpret_cast<const QualityReq*>(pr.dev);
  qp.logits = d_logits;
  qp.lse = d_lse;
  qp.list = d_list;
  qp.p = static_cast<float*>(d_ws);
  qp.top = d_top;
  qp.coverage = d_coverage;
  qp.recall = d_recall;
  qp.Hq = num_qo_heads;
  qp.G = num_qo_heads / num_kv_heads;
  qp.row = row;
  qp.T = top_t;
  hipError_t e = launch_quality(qp, B * num_qo_heads, quality_smem_bytes(max_len), st);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("quality launch: ") + hipGetErrorString(e));
  e = launch_release(pr.done_dev, pr.seq, st);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, std::string("release launch: ") + hipGetErrorString(e));
  arm_plan(pr, 1u);
  return SPA_OK;
}

}  // extern "C"
