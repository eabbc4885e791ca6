// kvcache.cpp -- include/spa_kvcache.h: block copies between the device KV
// pools and pinned host chunks on a copy stream, and the host-side block
// manager that plans them.
//
// Review of SparseSpec, 核心方法 / "Dynamic KV-Cache manager" (chunk-wise
// asynchronous offload to host, first in first out, offloaded requests
// scheduled first when memory frees up) and 关键观察, observation 5.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "spa_error.h"
#include "spa_kvcache.h"

namespace {

int32_t fail(int32_t code, const std::string& msg) { return spa::set_error(code, msg); }

// ---------------------------------------------------------------------------
// block copies
// ---------------------------------------------------------------------------
size_t block_bytes_of(const spa_layout* l, int32_t block_slots) {
  if (!l || block_slots < 1 || l->num_kv_heads < 1 || (l->head_dim != 64 && l->head_dim != 128) ||
      (l->dtype != SPA_BF16 && l->dtype != SPA_F32) || l->num_slots < 1)
    return 0;
  const size_t esz = l->dtype == SPA_BF16 ? 2 : 4;
  return (size_t)block_slots * (size_t)l->num_kv_heads * (size_t)l->head_dim * esz;
}

bool pinned(const void* p) {
  void* d = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void*>(p), 0);
  if (e != hipSuccess || !d) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

// Checks the move list; on success fills the runs (first index, length) of
// pairs whose blocks and chunks both ascend by one.
int32_t check_moves(const spa_layout* l, int32_t block_slots, int32_t n, const int32_t* blk,
                    const int32_t* chk, const void* dk, const void* dv, const void* hk,
                    const void* hv, size_t arena_bytes, size_t* bb,
                    std::vector<std::pair<int32_t, int32_t>>* runs) {
  *bb = block_bytes_of(l, block_slots);
  if (*bb == 0) return fail(SPA_ERR_INVALID_ARG, "kv copy: invalid layout or block_slots");
  if (n < 0) return fail(SPA_ERR_INVALID_ARG, "kv copy: n < 0");
  if (n == 0) return SPA_OK;
  if (!blk || !chk || !dk || !dv || !hk || !hv)
    return fail(SPA_ERR_INVALID_ARG, "kv copy: NULL block list, chunk list, pool or arena");
  const int64_t nblocks = l->num_slots / block_slots;
  const int64_t nchunks = (int64_t)(arena_bytes / *bb);
  std::vector<int32_t> a(blk, blk + n), c(chk, chk + n);
  for (int32_t i = 0; i < n; ++i) {
    if (a[i] < 0 || a[i] >= nblocks)
      return fail(SPA_ERR_INVALID_ARG, "kv copy: block " + std::to_string(a[i]) + " outside [0, " +
                                           std::to_string(nblocks) + ")");
    if (c[i] < 0 || c[i] >= nchunks)
      return fail(SPA_ERR_INVALID_ARG, "kv copy: chunk " + std::to_string(c[i]) +
                                           " outside the arenas (" + std::to_string(nchunks) +
                                           " chunks)");
  }
  std::sort(a.begin(), a.end());
  std::sort(c.begin(), c.end());
  if (std::adjacent_find(a.begin(), a.end()) != a.end())
    return fail(SPA_ERR_INVALID_ARG, "kv copy: a block appears twice");
  if (std::adjacent_find(c.begin(), c.end()) != c.end())
    return fail(SPA_ERR_INVALID_ARG, "kv copy: a chunk appears twice");
  if (!pinned(hk) || !pinned(hv))
    return fail(SPA_ERR_INVALID_ARG, "kv copy: the host arenas must be pinned host memory");
  runs->clear();
  int32_t s = 0;
  for (int32_t i = 1; i <= n; ++i) {
    if (i == n || blk[i] != blk[i - 1] + 1 || chk[i] != chk[i - 1] + 1) {
      runs->push_back({s, i - s});
      s = i;
    }
  }
  return SPA_OK;
}

int32_t copy_runs(bool to_host, const int32_t* blk, const int32_t* chk, size_t bb,
                  const std::vector<std::pair<int32_t, int32_t>>& runs, char* dk, char* dv,
                  char* hk, char* hv, void* wait_event, void* done_event, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (wait_event) e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(wait_event), 0);
  for (size_t i = 0; i < runs.size() && e == hipSuccess; ++i) {
    const int32_t f = runs[i].first, len = runs[i].second;
    const size_t doff = (size_t)blk[f] * bb, hoff = (size_t)chk[f] * bb, bytes = (size_t)len * bb;
    if (to_host) {
      e = hipMemcpyAsync(hk + hoff, dk + doff, bytes, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipMemcpyAsync(hv + hoff, dv + doff, bytes, hipMemcpyDeviceToHost, s);
    } else {
      e = hipMemcpyAsync(dk + doff, hk + hoff, bytes, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipMemcpyAsync(dv + doff, hv + hoff, bytes, hipMemcpyHostToDevice, s);
    }
  }
  if (e == hipSuccess && done_event) e = hipEventRecord(static_cast<hipEvent_t>(done_event), s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(SPA_ERR_HIP, std::string("kv copy: ") + hipGetErrorString(e));
  }
  return SPA_OK;
}

// ---------------------------------------------------------------------------
// block manager
// ---------------------------------------------------------------------------
constexpr uint64_t KVM_MAGIC = 0x53504b564d475231ull;  // "SPKVMGR1"
enum : int8_t { NONE = 0, RESIDENT = 1, OFFLOADED = 2 };

struct Header {
  uint64_t magic;
  spa_kvm_config cfg;
  int64_t admit_seq, off_seq;
  int32_t dev_cursor, host_cursor;
  spa_kvm_stats stats;
  // array offsets
  size_t where, nblk, admit, offq, mark, blocks, dev_used, host_used, total;
};

size_t align64(size_t x) { return (x + 63) / 64 * 64; }

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}
template <typename T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

int32_t check_config(const spa_kvm_config* c) {
  if (!c) return fail(SPA_ERR_INVALID_ARG, "kvm: config is NULL");
  if (c->dev_blocks < 1 || c->host_chunks < 0 || c->block_slots < 1 || c->max_requests < 1 ||
      c->max_blocks < 1)
    return fail(SPA_ERR_INVALID_ARG, "kvm: dev_blocks, block_slots, max_requests and max_blocks "
                                     "must be positive, host_chunks non-negative");
  if ((int64_t)c->max_requests * c->max_blocks > ((int64_t)1 << 31))
    return fail(SPA_ERR_INVALID_ARG, "kvm: max_requests * max_blocks above 2^31");
  return SPA_OK;
}

Header layout(const spa_kvm_config& c) {
  Header h;
  std::memset(&h, 0, sizeof h);
  h.cfg = c;
  const size_t R = (size_t)c.max_requests;
  size_t o = align64(sizeof(Header));
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = align64(o + bytes);
    return r;
  };
  h.where = take(R);
  h.nblk = take(R * 4);
  h.admit = take(R * 8);
  h.offq = take(R * 8);
  h.mark = take(R);
  h.blocks = take(R * (size_t)c.max_blocks * 4);
  h.dev_used = take(((size_t)c.dev_blocks + 63) / 64 * 8);
  h.host_used = take(((size_t)c.host_chunks + 63) / 64 * 8 + 8);
  h.total = o;
  return h;
}

Header* header(void* st) {
  Header* h = static_cast<Header*>(st);
  return (h && h->magic == KVM_MAGIC) ? h : nullptr;
}
const Header* header(const void* st) {
  const Header* h = static_cast<const Header*>(st);
  return (h && h->magic == KVM_MAGIC) ? h : nullptr;
}

// The first clear bit at or after `cursor` (wrapping), set; -1 if none.
int32_t take_bit(uint64_t* bits, int32_t n, int32_t* cursor) {
  const int32_t words = (n + 63) / 64;
  int32_t i = (*cursor >= 0 && *cursor < n) ? *cursor : 0;
  for (int32_t scanned = 0; scanned <= words; ++scanned) {
    const int32_t w = i / 64;
    uint64_t free = ~bits[w] & (~0ull << (i % 64));
    if (w == words - 1 && n % 64) free &= (1ull << (n % 64)) - 1;
    if (free) {
      const int32_t b = w * 64 + __builtin_ctzll(free);
      bits[w] |= 1ull << (b % 64);
      *cursor = b + 1 < n ? b + 1 : 0;
      return b;
    }
    i = (w + 1 < words) ? (w + 1) * 64 : 0;
  }
  return -1;
}

void clear_bit(uint64_t* bits, int32_t b) { bits[b / 64] &= ~(1ull << (b % 64)); }

}  // namespace

extern "C" {

size_t spa_kv_block_bytes(const spa_layout* layout, int32_t block_slots) {
  return block_bytes_of(layout, block_slots);
}

int32_t spa_kv_offload(const spa_layout* layout, int32_t block_slots, int32_t n,
                       const int32_t* h_dev_block, const int32_t* h_host_chunk,
                       const void* d_k_pool, const void* d_v_pool, void* h_k_arena,
                       void* h_v_arena, size_t arena_bytes, void* wait_event, void* done_event,
                       void* stream) {
  size_t bb = 0;
  std::vector<std::pair<int32_t, int32_t>> runs;
  int32_t rc = check_moves(layout, block_slots, n, h_dev_block, h_host_chunk, d_k_pool, d_v_pool,
                           h_k_arena, h_v_arena, arena_bytes, &bb, &runs);
  if (rc) return rc;
  return copy_runs(true, h_dev_block, h_host_chunk, bb, runs,
                   const_cast<char*>(static_cast<const char*>(d_k_pool)),
                   const_cast<char*>(static_cast<const char*>(d_v_pool)),
                   static_cast<char*>(h_k_arena), static_cast<char*>(h_v_arena), wait_event,
                   done_event, stream);
}

int32_t spa_kv_prefetch(const spa_layout* layout, int32_t block_slots, int32_t n,
                        const int32_t* h_host_chunk, const int32_t* h_dev_block,
                        const void* h_k_arena, const void* h_v_arena, size_t arena_bytes,
                        void* d_k_pool, void* d_v_pool, void* wait_event, void* done_event,
                        void* stream) {
  size_t bb = 0;
  std::vector<std::pair<int32_t, int32_t>> runs;
  int32_t rc = check_moves(layout, block_slots, n, h_dev_block, h_host_chunk, d_k_pool, d_v_pool,
                           h_k_arena, h_v_arena, arena_bytes, &bb, &runs);
  if (rc) return rc;
  return copy_runs(false, h_dev_block, h_host_chunk, bb, runs, static_cast<char*>(d_k_pool),
                   static_cast<char*>(d_v_pool),
                   const_cast<char*>(static_cast<const char*>(h_k_arena)),
                   const_cast<char*>(static_cast<const char*>(h_v_arena)), wait_event,
                   done_event, stream);
}

size_t spa_kvm_bytes(const spa_kvm_config* cfg) {
  if (check_config(cfg)) return 0;
  return layout(*cfg).total;
}

int32_t spa_kvm_init(void* state, size_t bytes, const spa_kvm_config* cfg) {
  const int32_t rc = check_config(cfg);
  if (rc) return rc;
  if (!state || (reinterpret_cast<uintptr_t>(state) & 63) != 0)
    return fail(SPA_ERR_INVALID_ARG, "kvm: state must be non-NULL and 64-byte aligned");
  const Header h0 = layout(*cfg);
  if (bytes < h0.total)
    return fail(SPA_ERR_INVALID_ARG, "kvm: state of " + std::to_string(bytes) + " bytes, need " +
                                         std::to_string(h0.total));
  std::memset(state, 0, h0.total);
  Header* h = static_cast<Header*>(state);
  *h = h0;
  h->magic = KVM_MAGIC;
  h->stats.free_dev_blocks = cfg->dev_blocks;
  h->stats.free_host_chunks = cfg->host_chunks;
  return SPA_OK;
}

int32_t spa_kvm_reserve(void* state, int32_t req, int32_t len) {
  Header* h = header(state);
  if (!h) return fail(SPA_ERR_INVALID_ARG, "kvm: state not initialised");
  const spa_kvm_config& c = h->cfg;
  if (req < 0 || req >= c.max_requests || len < 0)
    return fail(SPA_ERR_INVALID_ARG, "kvm: request id outside [0, max_requests) or len < 0");
  int8_t* where = at<int8_t>(state, h->where);
  int32_t* nblk = at<int32_t>(state, h->nblk);
  if (where[req] == OFFLOADED)
    return fail(SPA_ERR_INVALID_ARG, "kvm: request " + std::to_string(req) + " is offloaded");
  const int64_t need = ((int64_t)len + c.block_slots - 1) / c.block_slots;
  if (need > c.max_blocks)
    return fail(SPA_ERR_INVALID_ARG, "kvm: " + std::to_string(len) + " positions exceed max_blocks");
  const int32_t m = (int32_t)need - nblk[req];
  if (m <= 0) return SPA_OK;
  if (m > h->stats.free_dev_blocks)
    return fail(SPA_ERR_KV_FULL, "kvm: " + std::to_string(m) + " device blocks needed, " +
                                     std::to_string(h->stats.free_dev_blocks) + " free");
  if (where[req] == NONE) {
    where[req] = RESIDENT;
    at<int64_t>(state, h->admit)[req] = ++h->admit_seq;
    h->stats.resident += 1;
  }
  int32_t* blocks = at<int32_t>(state, h->blocks) + (size_t)req * c.max_blocks;
  uint64_t* used = at<uint64_t>(state, h->dev_used);
  for (int32_t i = 0; i < m; ++i) blocks[nblk[req] + i] = take_bit(used, c.dev_blocks, &h->dev_cursor);
  nblk[req] += m;
  h->stats.free_dev_blocks -= m;
  return SPA_OK;
}

int32_t spa_kvm_release(void* state, int32_t req) {
  Header* h = header(state);
  if (!h) return fail(SPA_ERR_INVALID_ARG, "kvm: state not initialised");
  const spa_kvm_config& c = h->cfg;
  if (req < 0 || req >= c.max_requests) return fail(SPA_ERR_INVALID_ARG, "kvm: request id");
  int8_t* where = at<int8_t>(state, h->where);
  int32_t* nblk = at<int32_t>(state, h->nblk);
  const int32_t* blocks = at<int32_t>(state, h->blocks) + (size_t)req * c.max_blocks;
  if (where[req] == RESIDENT) {
    uint64_t* used = at<uint64_t>(state, h->dev_used);
    for (int32_t i = 0; i < nblk[req]; ++i) clear_bit(used, blocks[i]);
    h->stats.free_dev_blocks += nblk[req];
    h->stats.resident -= 1;
  } else if (where[req] == OFFLOADED) {
    uint64_t* used = at<uint64_t>(state, h->host_used);
    for (int32_t i = 0; i < nblk[req]; ++i) clear_bit(used, blocks[i]);
    h->stats.free_host_chunks += nblk[req];
    h->stats.offloaded -= 1;
  }
  where[req] = NONE;
  nblk[req] = 0;
  return SPA_OK;
}

int32_t spa_kvm_plan_offload(void* state, int32_t need_free, const int32_t* h_keep, int32_t n_keep,
                             int32_t cap, int32_t* dev_block, int32_t* host_chunk,
                             int32_t* n_moves, int32_t* reqs, int32_t* n_reqs) {
  Header* h = header(state);
  if (!h || !n_moves || !n_reqs || (cap > 0 && (!dev_block || !host_chunk)) || !reqs ||
      n_keep < 0 || (n_keep > 0 && !h_keep) || cap < 0)
    return fail(SPA_ERR_INVALID_ARG, "kvm: plan_offload arguments");
  const spa_kvm_config& c = h->cfg;
  int8_t* where = at<int8_t>(state, h->where);
  int32_t* nblk = at<int32_t>(state, h->nblk);
  const int64_t* admit = at<int64_t>(state, h->admit);
  int64_t* offq = at<int64_t>(state, h->offq);
  uint8_t* mark = at<uint8_t>(state, h->mark);
  int32_t* blocks_all = at<int32_t>(state, h->blocks);
  uint64_t* dev_used = at<uint64_t>(state, h->dev_used);
  uint64_t* host_used = at<uint64_t>(state, h->host_used);
  for (int32_t i = 0; i < n_keep; ++i) {
    if (h_keep[i] < 0 || h_keep[i] >= c.max_requests)
      return fail(SPA_ERR_INVALID_ARG, "kvm: keep list holds an invalid request id");
  }
  std::memset(mark, 0, (size_t)c.max_requests);
  for (int32_t i = 0; i < n_keep; ++i) mark[h_keep[i]] = 1;
  int32_t moves = 0, nr = 0;
  while (h->stats.free_dev_blocks < need_free) {
    int32_t v = -1;
    for (int32_t r = 0; r < c.max_requests; ++r)
      if (where[r] == RESIDENT && !mark[r] && nblk[r] > 0 && (v < 0 || admit[r] > admit[v])) v = r;
    if (v < 0) break;
    const int32_t m = nblk[v];
    if (moves + m > cap || m > h->stats.free_host_chunks) break;
    int32_t* blocks = blocks_all + (size_t)v * c.max_blocks;
    for (int32_t i = 0; i < m; ++i) {
      const int32_t chunk = take_bit(host_used, c.host_chunks, &h->host_cursor);
      dev_block[moves] = blocks[i];
      host_chunk[moves] = chunk;
      clear_bit(dev_used, blocks[i]);
      blocks[i] = chunk;
      ++moves;
    }
    where[v] = OFFLOADED;
    offq[v] = ++h->off_seq;
    mark[v] = 1;
    reqs[nr++] = v;
    h->stats.free_dev_blocks += m;
    h->stats.free_host_chunks -= m;
    h->stats.resident -= 1;
    h->stats.offloaded += 1;
    h->stats.offloads += 1;
    h->stats.blocks_offloaded += m;
  }
  *n_moves = moves;
  *n_reqs = nr;
  return SPA_OK;
}

int32_t spa_kvm_plan_prefetch(void* state, int32_t keep_free, int32_t cap, int32_t* host_chunk,
                              int32_t* dev_block, int32_t* n_moves, int32_t* reqs,
                              int32_t* n_reqs) {
  Header* h = header(state);
  if (!h || !n_moves || !n_reqs || !reqs || cap < 0 || (cap > 0 && (!dev_block || !host_chunk)) ||
      keep_free < 0)
    return fail(SPA_ERR_INVALID_ARG, "kvm: plan_prefetch arguments");
  const spa_kvm_config& c = h->cfg;
  int8_t* where = at<int8_t>(state, h->where);
  const int32_t* nblk = at<int32_t>(state, h->nblk);
  const int64_t* offq = at<int64_t>(state, h->offq);
  int32_t* blocks_all = at<int32_t>(state, h->blocks);
  uint64_t* dev_used = at<uint64_t>(state, h->dev_used);
  uint64_t* host_used = at<uint64_t>(state, h->host_used);
  int32_t moves = 0, nr = 0;
  for (;;) {
    int32_t v = -1;
    for (int32_t r = 0; r < c.max_requests; ++r)
      if (where[r] == OFFLOADED && (v < 0 || offq[r] < offq[v])) v = r;
    if (v < 0) break;
    const int32_t m = nblk[v];
    if (h->stats.free_dev_blocks - m < keep_free || moves + m > cap) break;
    int32_t* blocks = blocks_all + (size_t)v * c.max_blocks;
    for (int32_t i = 0; i < m; ++i) {
      const int32_t b = take_bit(dev_used, c.dev_blocks, &h->dev_cursor);
      host_chunk[moves] = blocks[i];
      dev_block[moves] = b;
      clear_bit(host_used, blocks[i]);
      blocks[i] = b;
      ++moves;
    }
    where[v] = RESIDENT;
    reqs[nr++] = v;
    h->stats.free_dev_blocks -= m;
    h->stats.free_host_chunks += m;
    h->stats.resident += 1;
    h->stats.offloaded -= 1;
    h->stats.prefetches += 1;
    h->stats.blocks_prefetched += m;
  }
  *n_moves = moves;
  *n_reqs = nr;
  return SPA_OK;
}

int32_t spa_kvm_page_row(const void* state, int32_t req, int32_t len, int32_t* out) {
  const Header* h = header(state);
  if (!h || !out) return fail(SPA_ERR_INVALID_ARG, "kvm: state not initialised or out is NULL");
  const spa_kvm_config& c = h->cfg;
  if (req < 0 || req >= c.max_requests) return fail(SPA_ERR_INVALID_ARG, "kvm: request id");
  const int8_t* where = at<int8_t>(state, h->where);
  const int32_t* nblk = at<int32_t>(state, h->nblk);
  if (where[req] != RESIDENT)
    return fail(SPA_ERR_INVALID_ARG, "kvm: request " + std::to_string(req) + " is not resident");
  if (len < 0 || (int64_t)len > (int64_t)nblk[req] * c.block_slots)
    return fail(SPA_ERR_INVALID_ARG, "kvm: len beyond the request's blocks");
  const int32_t* blocks = at<int32_t>(state, h->blocks) + (size_t)req * c.max_blocks;
  for (int32_t j = 0; j < len; ++j)
    out[j] = blocks[j / c.block_slots] * c.block_slots + j % c.block_slots;
  return SPA_OK;
}

int32_t spa_kvm_where(const void* state, int32_t req) {
  const Header* h = header(state);
  if (!h) {
    fail(SPA_ERR_INVALID_ARG, "kvm: state not initialised");
    return -1;
  }
  if (req < 0 || req >= h->cfg.max_requests) return -1;
  return at<int8_t>(state, h->where)[req];
}

int32_t spa_kvm_stats_read(const void* state, spa_kvm_stats* out) {
  const Header* h = header(state);
  if (!h || !out) return fail(SPA_ERR_INVALID_ARG, "kvm: state not initialised or out is NULL");
  *out = h->stats;
  return SPA_OK;
}

}  // extern "C"
