/*
 * spa_probe.h -- libspa_probe: the attainable HBM bandwidth of the decode
 * attention launch's access mix on one GPU, for judging how close the launch
 * runs to what the memory system delivers for that mix (as opposed to the
 * 8 TB/s peak of plain sequential streaming).
 *
 * The attention launch reads KV rows of head_dim bf16 elements (256 bytes at
 * head_dim 128) from slots scattered over the pool (page size 1), K and V for
 * every position of a (request, KV head) work item, and writes verify logits
 * sequentially.  spa_probe_ceiling replays that mix without the arithmetic:
 * work unit c covers 32 positions of KV head c mod H_kv, reads the K row and
 * the V row (256 bytes each) of each position's slot, then stores
 * write_bytes_per_chunk bytes of sequential output that depend on what it read.
 * Slots are a hash of (c, position) in [0, num_slots) when `random` is set
 * (the launch's scattered rows), else 32 consecutive slots per unit.  KV reads
 * carry the non-temporal hint, as the launch's do.  `depth` units are loaded
 * before any is consumed (bytes in flight per workgroup: depth * 16 KiB).
 */
#ifndef SPA_PROBE_H_
#define SPA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* d_k, d_v: device pools [num_slots][num_kv_heads][128] bf16 (256-byte rows),
 * read only.  chunks: work units (32 positions each).  depth: 1, 2 or 4.
 * d_out: device buffer of out_bytes bytes, a multiple of write_bytes_per_chunk
 * (0..4096, a multiple of 16; 0 writes nothing, d_out may then be NULL); unit
 * c writes at (c * write_bytes_per_chunk) mod out_bytes.  grid: workgroups of
 * 256 threads (each loops over units).  d_sink: one device uint32 written only
 * in the rare case that a workgroup's XOR of everything it read is a fixed
 * constant (it keeps the loads alive).  Returns 0, or 1 for an invalid
 * argument, 2 for a launch error; enqueued on `stream` (NULL: default). */
int32_t spa_probe_ceiling(const void* d_k, const void* d_v, int64_t num_slots,
                          int32_t num_kv_heads, int64_t chunks, int32_t random, int32_t depth,
                          void* d_out, int64_t out_bytes, int32_t write_bytes_per_chunk,
                          int32_t grid, uint32_t* d_sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPA_PROBE_H_ */
