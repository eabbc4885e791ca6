/*
 * spa_kvcache.h -- chunk-wise asynchronous host offload and prefetch of the
 * KV pools of spa.h, and a host-side block manager that decides what moves.
 *
 * Pages: "SparseSpec-MLSys26" review (awesome-system-papers), 核心方法,
 * "Dynamic KV-Cache manager" (admit requests aggressively; when device KV
 * memory runs out, move KV to host memory chunk by chunk and asynchronously,
 * first in first out for fairness, and schedule offloaded requests first once
 * device memory frees up; the moves cost about 0.5% of cycle time) and
 * 关键观察, observation 5 (about 18 MB of new KV per step for Qwen3-8B at
 * batch 128, which an asynchronous host link can carry alongside the GPU's
 * work).
 *
 * Blocks and chunks.  The pools ([num_slots][H_kv][d], spa.h) are cut into
 * blocks of block_slots consecutive slots: block b holds slots
 * b*block_slots .. (b+1)*block_slots - 1, which are block_bytes =
 * block_slots * H_kv * d * esz contiguous bytes of each pool.  Attention keeps
 * page size 1 (any slot per position); the block manager below places
 * position j of a request at slot blk[j / block_slots] * block_slots +
 * j % block_slots, so a request moves block by block.  A host chunk is
 * block_bytes of caller-owned pinned host memory per pool: two arenas, one for
 * K and one for V, each [host_chunks][block_bytes], allocated with
 * hipHostMalloc (or a pinned torch tensor).  The copies run on the copy
 * engines, so attention kernels keep every compute unit meanwhile.
 */
#ifndef SPA_KVCACHE_H_
#define SPA_KVCACHE_H_

#include <stddef.h>
#include <stdint.h>

#include "spa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of one block in one pool (0 for an invalid layout or block_slots < 1). */
size_t spa_kv_block_bytes(const spa_layout* layout, int32_t block_slots);

/* Offload: copies device block h_dev_block[i] of both pools into host chunk
 * h_host_chunk[i] of the two arenas, for i < n, enqueued on `stream` (the
 * caller's copy stream) after `wait_event` (if not NULL, e.g. recorded after
 * the last kernel that reads or writes those blocks) and followed by
 * `done_event` (if not NULL): once it has completed, the blocks may be
 * reused and the chunks read.  Pairs whose blocks and chunks both ascend by
 * one are merged into one copy per pool.  Blocks must be distinct and lie in
 * [0, num_slots / block_slots); chunks distinct and inside both arenas
 * (arena_bytes each, pinned host memory, checked).  Host-side errors
 * (SPA_ERR_INVALID_ARG) enqueue nothing. */
int32_t spa_kv_offload(const spa_layout* layout, int32_t block_slots, int32_t n,
                       const int32_t* h_dev_block, const int32_t* h_host_chunk,
                       const void* d_k_pool, const void* d_v_pool, void* h_k_arena,
                       void* h_v_arena, size_t arena_bytes, void* wait_event,
                       void* done_event, void* stream);

/* Prefetch: copies host chunk h_host_chunk[i] into device block
 * h_dev_block[i] of both pools, for i < n; same rules.  Once done_event has
 * completed, attention may read the blocks and the chunks may be reused. */
int32_t spa_kv_prefetch(const spa_layout* layout, int32_t block_slots, int32_t n,
                        const int32_t* h_host_chunk, const int32_t* h_dev_block,
                        const void* h_k_arena, const void* h_v_arena, size_t arena_bytes,
                        void* d_k_pool, void* d_v_pool, void* wait_event, void* done_event,
                        void* stream);

/* Block manager: which device blocks and host chunks each request holds.
 * Requests are ids 0..max_requests-1.  A request is admitted by its first
 * reserve; it is resident (its blocks on the device) or offloaded (its
 * blocks in host chunks).  Offload victims are the resident requests admitted
 * last (the oldest requests keep their memory); offloaded requests come back
 * in the order they left (first in, first out).  The manager only plans: the
 * caller issues the copies (spa_kv_offload / spa_kv_prefetch) for the moves
 * it returns, orders them against the kernels with events, and rewrites the
 * page-table rows of requests that came back (spa_kvm_page_row).  Blocks an
 * offload plan frees may be handed out again at once: the caller must not
 * write them before that offload's done_event.  State: spa_kvm_bytes(cfg)
 * bytes of host memory, 64-byte aligned, owned by the caller; the manager
 * allocates nothing.  Not thread-safe for one state. */
typedef struct {
  int32_t dev_blocks;     /* device blocks the pools hold (num_slots / block_slots or fewer) */
  int32_t host_chunks;    /* host chunks in the arenas                                  */
  int32_t block_slots;    /* slots per block                                            */
  int32_t max_requests;   /* request ids 0..max_requests-1                              */
  int32_t max_blocks;     /* blocks one request may hold                                */
} spa_kvm_config;

typedef struct {
  int32_t resident, offloaded;            /* requests                               */
  int32_t free_dev_blocks, free_host_chunks;
  int64_t offloads, prefetches;           /* requests moved, since init              */
  int64_t blocks_offloaded, blocks_prefetched;
} spa_kvm_stats;

size_t spa_kvm_bytes(const spa_kvm_config* cfg);
int32_t spa_kvm_init(void* state, size_t bytes, const spa_kvm_config* cfg);

/* Gives request `req` blocks for `len` positions (admitting it if it holds
 * none): the lowest free device blocks at or after the last one handed out.
 * SPA_ERR_KV_FULL (nothing changes) when the free device blocks do not
 * suffice; SPA_ERR_INVALID_ARG for an offloaded request or len beyond
 * max_blocks * block_slots. */
int32_t spa_kvm_reserve(void* state, int32_t req, int32_t len);

/* Frees everything the request holds (it finished); a no-op for a request
 * that holds nothing. */
int32_t spa_kvm_release(void* state, int32_t req);

/* Plans offloading whole resident requests, admitted last first, until at
 * least `need_free` device blocks are free, skipping the n_keep requests of
 * h_keep (those about to run).  Writes the moves (dev_block[i] ->
 * host_chunk[i], at most cap) and the requests moved (at most max_requests);
 * a request is moved only if all of its moves fit in `cap` and in the free host
 * chunks.  Returns SPA_OK with *n_moves = 0 when nothing needs to or can move. */
int32_t spa_kvm_plan_offload(void* state, int32_t need_free, const int32_t* h_keep, int32_t n_keep,
                             int32_t cap, int32_t* dev_block, int32_t* host_chunk,
                             int32_t* n_moves, int32_t* reqs, int32_t* n_reqs);

/* Plans bringing offloaded requests back, first offloaded first, while each
 * one's blocks fit in the free device blocks beyond `keep_free`; stops at the
 * first that does not fit (the queue keeps its order).  Writes the moves
 * (host_chunk[i] -> dev_block[i], at most cap) and the requests. */
int32_t spa_kvm_plan_prefetch(void* state, int32_t keep_free, int32_t cap, int32_t* host_chunk,
                              int32_t* dev_block, int32_t* n_moves, int32_t* reqs,
                              int32_t* n_reqs);

/* Page-table row of a resident request for its first len positions:
 * out[j] = slot of position j. */
int32_t spa_kvm_page_row(const void* state, int32_t req, int32_t len, int32_t* out);

/* 1 resident, 2 offloaded, 0 holds nothing; negative for an invalid call. */
int32_t spa_kvm_where(const void* state, int32_t req);

int32_t spa_kvm_stats_read(const void* state, spa_kvm_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* SPA_KVCACHE_H_ */
