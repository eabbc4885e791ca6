// probe.hip -- libspa_probe: replays the decode attention launch's HBM access
// mix (scattered 256-byte K and V rows, non-temporal, plus dependent
// sequential stores) without its arithmetic, to measure the bandwidth that
// mix can attain on the device.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_probe.h"

namespace {

constexpr int ROW_BYTES = 256;         // one KV row: head_dim 128 in bf16
constexpr int UNIT_POS = 32;           // positions per unit (one attention tile)
constexpr int PIECES = 2 * UNIT_POS * ROW_BYTES / 16;  // 16-byte pieces per unit: 1024
constexpr int THREADS = 256;
constexpr int PER_THREAD = PIECES / THREADS;             // 4
constexpr uint32_t SINK_MAGIC = 0x5bd1e995u;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Piece j of thread t: row (t / 16) + 16 j of the unit's 64 rows (rows 0..31
// are K rows of positions 0..31, rows 32..63 the V rows), bytes 16 (t % 16)
// of the row; 16 consecutive lanes read one whole row.
template <int DEPTH>
__global__ __launch_bounds__(THREADS) void probe_kernel(const char* __restrict__ kp,
                                                        const char* __restrict__ vp,
                                                        int64_t num_slots, int32_t hkv,
                                                        int64_t chunks, int32_t random,
                                                        char* __restrict__ out, int64_t out_bytes,
                                                        int32_t wbytes, uint32_t* sink) {
  const int t = threadIdx.x;
  const int piece = t & 15;
  const int row0 = t >> 4;  // 0..15
  uint32_t acc = 0;
  for (int64_t c0 = (int64_t)blockIdx.x * DEPTH; c0 < chunks; c0 += (int64_t)gridDim.x * DEPTH) {
    u32x4 v[DEPTH][PER_THREAD];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int64_t c = c0 + u < chunks ? c0 + u : chunks - 1;
      const int64_t g = c % hkv;
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) {
        const int row = row0 + 16 * j;
        const int pos = row & (UNIT_POS - 1);
        const int64_t slot = random
            ? (int64_t)(mix32((uint32_t)(c * UNIT_POS + pos) * 2654435761u + 0x9e3779b9u) %
                        (uint64_t)num_slots)
            : ((c / hkv) * UNIT_POS + pos) % num_slots;
        const char* base = row < UNIT_POS ? kp : vp;
        const char* src = base + (slot * hkv + g) * ROW_BYTES + piece * 16;
        v[u][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      }
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      uint32_t x = 0;
#pragma unroll
      for (int j = 0; j < PER_THREAD; ++j) x ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
      acc ^= x;
      const int64_t c = c0 + u;
      if (c < chunks && t * 16 < wbytes) {
        const int64_t off = (c * wbytes) % out_bytes + t * 16;
        u32x4 o = {x, x + 1u, x + 2u, x + 3u};
        *reinterpret_cast<u32x4*>(out + off) = o;
      }
    }
  }
  if (acc == SINK_MAGIC) sink[0] = acc;
}

}  // namespace

extern "C" int32_t spa_probe_ceiling(const void* d_k, const void* d_v, int64_t num_slots,
                                     int32_t num_kv_heads, int64_t chunks, int32_t random,
                                     int32_t depth, void* d_out, int64_t out_bytes,
                                     int32_t write_bytes_per_chunk, int32_t grid, uint32_t* d_sink,
                                     void* stream) {
  if (!d_k || !d_v || !d_sink || num_slots < 1 || num_kv_heads < 1 || chunks < 0 || grid < 1)
    return 1;
  if (num_slots > ((int64_t)1 << 31)) return 1;
  const int32_t wb = write_bytes_per_chunk;
  if (wb < 0 || wb > THREADS * 16 || wb % 16 != 0) return 1;
  if (wb > 0 && (!d_out || out_bytes < wb || out_bytes % wb != 0)) return 1;
  if (chunks == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* k = static_cast<const char*>(d_k);
  const char* v = static_cast<const char*>(d_v);
  char* o = static_cast<char*>(d_out);
  const int64_t ob = wb > 0 ? out_bytes : 16;
  switch (depth) {
    case 1:
      probe_kernel<1><<<grid, THREADS, 0, s>>>(k, v, num_slots, num_kv_heads, chunks, random, o, ob,
                                               wb, d_sink);
      break;
    case 2:
      probe_kernel<2><<<grid, THREADS, 0, s>>>(k, v, num_slots, num_kv_heads, chunks, random, o, ob,
                                               wb, d_sink);
      break;
    case 4:
      probe_kernel<4><<<grid, THREADS, 0, s>>>(k, v, num_slots, num_kv_heads, chunks, random, o, ob,
                                               wb, d_sink);
      break;
    default:
      return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
