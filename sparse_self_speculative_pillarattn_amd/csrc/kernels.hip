// kernels.hip -- device code of libspa for gfx950 (CDNA4).
//
// A unified step is three launches on the caller's stream, five with rows
// longer than 32,768 scores (pages: the
// SparseSpec review, 核心方法 -> PillarAttn and "Unified batch scheduler +
// fused attention kernel"):
// attn_kernel    persistent workgroups draw plan items from a ticket counter:
//                a verify item (request r, KV head g, a chunk of positions) or a
//                draft item (r, one or several KV heads, a chunk of the index
//                list).  In bf16 both run the wave-specialised MFMA tile: a
//                producer wave streams K/V rows into a 4-stage LDS ring with
//                global->LDS loads, consumer waves compute S = K Q^T and
//                O = P V; verify tiles dump their logits.  fp32 runs the VALU
//                gather tile.  Outputs are final when (r, g) is one chunk,
//                split-K partials otherwise.  No workgroup waits for another.
// attn_kernel_draft  the same loop for the draft items of a step whose drafts
//                run as a second launch on a side stream (the overlap option).
// post_kernel    split-K log-sum-exp merges, and the exact scores
//                exp(logit - LSE) averaged over the draft rows and the GQA group
//                in 1024-position items, counted into a per-(r, g) histogram.
// select_kernel  one workgroup per verify (r, g): the top-K by a radix select
//                seeded by that histogram, written ascending.
// select_count_kernel, select_chunk_kernel  rows longer than 32,768 scores,
//                one workgroup per 8192-score chunk: counts above the
//                histogram's boundary bin and that bin's keys, then each
//                chunk's positions written at its offset in the list.
// release_kernel one thread that marks a plan buffer free when no other launch
//                of the call does.
// recall_kernel, quality_kernel  the neighbours of the step: index lists with
//                sinks and recent positions appended, and the coverage / recall
//                of lists against one query row's exact attention.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <mutex>
#include <vector>

#include "spa_kernels.h"
#include "spa_plan.h"

namespace spa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));  // 16 bytes at a 4-byte boundary

constexpr float LOG2E = 1.4426950408889634f;
#define NEG_INF (-__builtin_inff())

__device__ __forceinline__ uint32_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int64_t clamp_slot(int32_t s, int64_t n) {
  return s < 0 ? 0 : (s >= n ? n - 1 : (int64_t)s);
}

template <typename T>
struct Piece;
template <>
struct Piece<uint16_t> {  // bf16: 8 elements per 16 bytes
  static constexpr int E = 8;
  __device__ static void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Piece<float> {
  static constexpr int E = 4;
  __device__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

template <typename T>
__device__ __forceinline__ void store_out(T* dst, float v);
// Four consecutive elements widened to float (bf16 as raw uint16 bits).
template <typename T>
__device__ __forceinline__ float4 load4(const T* src);
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* src) {
  const uint2 v = *reinterpret_cast<const uint2*>(src);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
template <>
__device__ __forceinline__ float4 load4<float>(const float* src) {
  return *reinterpret_cast<const float4*>(src);
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* dst, float v) {
  *dst = (uint16_t)f2bf(v);
}
template <>
__device__ __forceinline__ void store_out<float>(float* dst, float v) {
  *dst = v;
}

// LDS chunk swizzle of the K tile: the 16 rows one MFMA operand read touches
// land on distinct bank groups.
template <int NCH>
__device__ __forceinline__ int kswz(int tau) {
  return ((tau & 3) | (((tau >> 3) & 3) << 2)) & (NCH - 1);
}

// DPP lane exchanges inside a row of 16 lanes (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each half row
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within each row

// Sum over groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32, 64); every
// lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<DPP_XOR1>(v);
  if constexpr (N >= 4) v += dpp<DPP_XOR2>(v);
  if constexpr (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp<DPP_MIRROR>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ==========================================================================
// Verify tile on MFMA (bf16), wave-specialised
//
// The last wave of the block is the producer: it streams the K and V rows of
// 32-token tiles from the paged pool straight into a ring of LDS stages with
// global->LDS loads.  It issues loads only, so it can wait for one tile while
// the next ones are still in flight.  The other waves are consumers, one per
// 16-row tile of rows rho = i*G + hh (query row i, head hh of the group):
//   S^T = K Q^T      16x16x32 MFMA over tokens 16t..16t+15 of the tile (t = 0, 1);
//                    A = K rows from LDS, B = Q^T in registers.  Lane (n, q)
//                    holds row n's scores of tokens 16t + 4q .. 16t + 4q + 3.
//   logits stored (each store writes 64 contiguous bytes per row); online
//   softmax in registers (two lane shuffles per row)
//   O^T += V^T P^T   B = P^T is the two S^T accumulators in bf16: contraction
//                    index 8q + j is token 4q + j (j < 4) or 16 + 4q + j - 4;
//                    A = V^T of the same tokens, read from the row-major V
//                    stage with the LDS transpose read.
// Consumers only read LDS, run MFMA and store.  One barrier per tile hands a
// stage from the producer to the consumers and, a tile later, back.
// ==========================================================================
constexpr int DMA_TT = TILE_TOKENS;  // tokens per stage
constexpr int DMA_STAGES = 4;  // LDS stages; DMA_STAGES - 1 tiles in flight

template <int D>
constexpr size_t dma_smem_bytes() {  // the stage ring; logits staging and slots follow it
  return (size_t)DMA_STAGES * 2 * DMA_TT * D * 2;
}
// Logits staging of one consumer wave: 16 rows of a tile, padded so that the
// column-major writes and the row-major reads are both free of bank conflicts.
constexpr int LSTG = DMA_TT + 4;  // floats per staged row
constexpr size_t logit_stage_bytes(int consumer_waves) { return (size_t)consumer_waves * 16 * LSTG * 4; }
constexpr int VERIFY_SLOT_BATCH = 8;  // verify slots a thread stages per round
constexpr int LIST_SLOT_BATCH = 4;    // draft list entries a thread stages per round

// LDS chunk swizzles of a stage.  K: the 16 consecutive rows one MFMA operand
// read touches land on distinct bank groups.  V: the eight rows (two 16-byte
// chunks each) of every half-wave transpose read land on distinct bank groups.
template <int NCH>
__device__ __forceinline__ int kswz_t(int tau) {
  return tau & (NCH - 1);
}
template <int NCH>
__device__ __forceinline__ int vswz(int tau) {
  return (2 * (tau & 7)) & (NCH - 1);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory to LDS: lane l's piece lands at
// dst + 16 l (dst is wave-uniform).
// KV rows are read once per step, so their loads carry the non-temporal hint
// (cache-policy bit NT): streaming them then leaves L2 and the Infinity Cache
// to the logits, which the post-pass reads back right after this launch.
constexpr int KV_LOAD_POLICY = 2;

__device__ __forceinline__ void load_lds16(const void* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, KV_LOAD_POLICY);
}

// 16 bytes of a KV row into registers, with the same streaming hint.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_kv16(const void* src) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Slots of one tile as the producer's lanes use them: lane l loads rows
// RPI j + l / NCH of the tile.
template <int D>
struct TileSlots {
  int v[DMA_TT * (D / 8) / 64];
};

template <int D>
__device__ __forceinline__ void read_tile_slots(TileSlots<D>& s, const int32_t* slots, int lane) {
  constexpr int RPI = 64 / (D / 8);
#pragma unroll
  for (int j = 0; j < DMA_TT / RPI; ++j) s.v[j] = slots[RPI * j + lane / (D / 8)];
}

template <int D>
__device__ __forceinline__ void issue_kv_tile(char* stage, const TileSlots<D>& s, const uint16_t* kp,
                                              const uint16_t* vp, int64_t rs, int lane) {
  constexpr int NCH = D / 8;         // 16-byte chunks per row
  constexpr int RPI = 64 / NCH;      // rows per load instruction
  constexpr int NI = DMA_TT / RPI;   // load instructions per tensor and tile
  constexpr int STAGE = DMA_TT * D * 2;
  const int sub = lane / NCH, pc = lane % NCH;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int tau = RPI * j + sub;
    const int64_t row = (int64_t)max(s.v[j], 0) * rs;  // a masked entry reads row 0
    load_lds16(kp + row + 8 * (pc ^ kswz_t<NCH>(tau)), stage + 1024 * j);
    load_lds16(vp + row + 8 * (pc ^ vswz<NCH>(tau)), stage + STAGE + 1024 * j);
  }
}

// Producer side of the per-tile barrier: wait until the awaited tile has
// landed in LDS, `after` tiles having been issued behind it, then meet the
// consumers.  A bare s_barrier: __syncthreads() would add a workgroup release
// fence, which drains every outstanding global->LDS load, not just this tile.
template <int PER_TILE>
__device__ __forceinline__ void producer_barrier(int after) {
  if (after >= 2)
    wait_vmcnt<2 * PER_TILE>();
  else if (after == 1)
    wait_vmcnt<PER_TILE>();
  else
    wait_vmcnt<0>();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// The chunk's slots are in LDS (slots[j], -1 for an entry that is masked)
// before the producer starts.  It issues only
// global->LDS loads, so partial vmcnt waits track its tiles exactly.
template <int D>
__device__ void dma_producer(const AttnParams& p, const Item& it, char* smem,
                                const int32_t* slots, int lane) {
  constexpr int NCH = D / 8;
  constexpr int PER_TILE = 2 * (DMA_TT * NCH / 64);  // load instructions per tile
  constexpr int STAGE2 = 2 * DMA_TT * D * 2;
  static_assert(DMA_STAGES == 3 || DMA_STAGES == 4, "the waits below allow at most two tiles behind");
  // a draft item may hold the lists of ng consecutive KV heads, tph tiles each
  const int tph = (it.end - it.begin + DMA_TT - 1) / DMA_TT;
  const int n = tph * max(1, it.ng);
  const uint16_t* kp0 = reinterpret_cast<const uint16_t*>(p.k_pool) + it.g * D;
  const uint16_t* vp0 = reinterpret_cast<const uint16_t*>(p.v_pool) + it.g * D;
  auto kp = [&](int t) { return kp0 + (t / tph) * D; };
  auto vp = [&](int t) { return vp0 + (t / tph) * D; };
  const int64_t rs = (int64_t)p.Hkv * D;
  // The slots of the next tile are read from LDS right after a tile is issued,
  // so that their latency (LDS is busy with the consumers' operand reads)
  // passes while the producer waits, not on the issue path.
  TileSlots<D> ts;
  read_tile_slots<D>(ts, slots, lane);
  for (int i = 0; i < min(n, DMA_STAGES - 1); ++i) {
    issue_kv_tile<D>(smem + i * STAGE2, ts, kp(i), vp(i), rs, lane);
    if (i + 1 < n) read_tile_slots<D>(ts, slots + (i + 1) * DMA_TT, lane);
  }
  producer_barrier<PER_TILE>(min(n, DMA_STAGES - 1) - 1);  // tile 0 ready
  for (int i = 0; i + 1 < n; ++i) {
    const int t = i + DMA_STAGES - 1;  // into the stage tile i-1 used
    if (t < n) {
      issue_kv_tile<D>(smem + (t % DMA_STAGES) * STAGE2, ts, kp(t), vp(t), rs, lane);
      if (t + 1 < n) read_tile_slots<D>(ts, slots + (t + 1) * DMA_TT, lane);
    }
    producer_barrier<PER_TILE>(min(n - 1, t) - (i + 1));  // tile i+1 ready
  }
}

// IS_LIST: a draft item (list tiles; masked entries) or a verify item
// (causal tiles; logits dumped).  Two instantiations, so that each kind's tile
// loop carries only its own masking and outputs.
template <int D, bool IS_LIST>
__device__ void dma_consumer(const AttnParams& p, const Item& it, char* smem,
                             const int32_t* slots, int wave, int lane, int* next_item,
                             uint32_t wrap) {
  constexpr bool is_list = IS_LIST;
  constexpr int NCH = D / 8;   // 16-byte chunks per K/V row
  constexpr int KS = D / 32;   // k-steps of S^T = K Q^T
  constexpr int DT = D / 16;   // d tiles of O^T
  constexpr int STAGE = DMA_TT * D * 2;
  const int G = p.G, Hq = p.Hq;
  const int rows_q = is_list ? 1 : p.k + 1;
  const int R = rows_q * G;
  const int L = it.L;
  const int jb = it.begin, je = it.end;
  const int n_tiles = (je - jb + DMA_TT - 1) / DMA_TT;  // per KV head
  const int ng = IS_LIST ? max(1, it.ng) : 1;  // KV heads of a packed draft item (1 otherwise)

  const int n = lane & 15, q4 = lane >> 4;
  const int rho = wave * 16 + n;
  const bool wave_active = wave * 16 < R;
  const bool row_ok = rho < R;
  const int qi = row_ok ? rho / G : 0;
  const int hh = row_ok ? rho % G : 0;
  int h = it.g * G + hh;

  bf16x8 qop[KS];
  float m_run = NEG_INF, l_run = 0.f;
  f32x4 oacc[DT];
  const int last_vis = is_list ? 0x7fffffff : L - rows_q + qi;
  float* lrow = is_list ? nullptr : p.logits + it.off + ((int64_t)qi * Hq + h) * L;
  const float sc = p.sm_scale;
  // Full tiles go out through this wave's LDS staging: 8 lanes then write
  // 128 contiguous bytes of one row (rows rA and rA + 8 of the wave).  A row
  // starts 16-byte aligned only when L and the logits offset are multiples of
  // 4; the 16-byte stores ask for 4-byte alignment (gfx950 serves them at any
  // 4-byte boundary).
  float* stg = reinterpret_cast<float*>(smem + dma_smem_bytes<D>()) + wave * 16 * LSTG;
  const int rA = lane >> 3, cA = 4 * (lane & 7);
  float* lA = nullptr;
  float* lB = nullptr;
  if (!is_list) {
    const int rho_a = wave * 16 + rA, rho_b = rho_a + 8;
    if (rho_a < R) lA = p.logits + it.off + ((int64_t)(rho_a / G) * Hq + it.g * G + rho_a % G) * L;
    if (rho_b < R) lB = p.logits + it.off + ((int64_t)(rho_b / G) * Hq + it.g * G + rho_b % G) * L;
  }

  // Transpose-read source rows of this lane: tokens 4 q + n / 4 and 16 more.
  // The lane supplies dims 4 (n % 4) .. + 3 of its 16-dim block.
  const int vrow0 = 4 * q4 + (n >> 2), vrow1 = vrow0 + 16;
  const int vcol = (n & 3);
  // causal limit of the earliest row of the request: every row sees a token
  // at or below it
  const int vis_all = L - rows_q;

  // the workgroup's next item, drawn by wave 0 two tiles before the end so
  // that the atomic's round trip passes under the last tiles
  uint32_t next = 0u;
  const int draw_at = max(ng * n_tiles - 2, 0);
  // query rows of a packed item's heads, staged in LDS with its slots
  const uint16_t* qst = reinterpret_cast<const uint16_t*>(slots + ng * n_tiles * DMA_TT);
  for (int hd = 0; hd < ng; ++hd) {
  h = (it.g + hd) * G + hh;
  {
    const uint16_t* qrow =
        ng > 1 ? qst + (int64_t)(hd * G + hh) * D
               : reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)(it.row0 + qi) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok) v = *reinterpret_cast<const uint4*>(qrow + 8 * (4 * s + q4));
      qop[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  m_run = NEG_INF;
  l_run = 0.f;
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n_tiles; ++i) {
    const int tt = hd * n_tiles + i;  // tile of the item: LDS stage and slots
    __syncthreads();  // tile tt ready (and tile tt-1 released)
    if (wave == 0 && lane == 0 && tt == draw_at)
      next = atomicInc(p.ticket, wrap);
    if (!wave_active) continue;
    const int t0 = jb + i * DMA_TT;
    const char* Ks = smem + (tt % DMA_STAGES) * 2 * STAGE;
    const char* Vs = Ks + STAGE;
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int tau = 16 * t + n;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + q4;
        const uint4 kv =
            *reinterpret_cast<const uint4*>(Ks + tau * NCH * 16 + 16 * (c ^ kswz_t<NCH>(tau)));
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qop[s],
                                                          sacc[t], 0, 0, 0);
      }
    }
    // full tile: every token inside the chunk and visible to every row (a
    // list tile is masked by the slots staged for it)
    const bool full = !is_list && t0 + DMA_TT <= je && t0 + DMA_TT - 1 <= vis_all;
    float v[2][4];
    float mx = NEG_INF;
    // V^T operand halves of masked list entries are zeroed before the P V
    // product: such an entry loads pool row 0 (whatever it holds), and its
    // exact zero weight would still turn an Inf or NaN there into NaN.
    // Element 4 t + e of a lane's V^T operand is token 16 t + 4 q + e.
    u32x4v vkeep = u32x4v{~0u, ~0u, ~0u, ~0u};
    if (full) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[t][e] = sacc[t][e] * sc;
          mx = fmaxf(mx, v[t][e]);
        }
      {
        // lane (n, q) holds row n's tokens 16 t + 4 q .. + 3; a wave's LDS
        // accesses complete in order, so the read-back needs no barrier
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<float4*>(stg + n * LSTG + 16 * t + 4 * q4) =
              make_float4(v[t][0], v[t][1], v[t][2], v[t][3]);
        const f32x4 va = *reinterpret_cast<const f32x4*>(stg + rA * LSTG + cA);
        const f32x4 vb = *reinterpret_cast<const f32x4*>(stg + (rA + 8) * LSTG + cA);
        if (lA) *reinterpret_cast<f32x4u*>(lA + t0 + cA) = va;
        if (lB) *reinterpret_cast<f32x4u*>(lB + t0 + cA) = vb;
      }
    } else {
      int ok[2][4];
      if (is_list) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int4 sv = *reinterpret_cast<const int4*>(slots + tt * DMA_TT + 16 * t + 4 * q4);
          ok[t][0] = sv.x >= 0;
          ok[t][1] = sv.y >= 0;
          ok[t][2] = sv.z >= 0;
          ok[t][3] = sv.w >= 0;
          vkeep[2 * t] = (ok[t][0] ? 0x0000ffffu : 0u) | (ok[t][1] ? 0xffff0000u : 0u);
          vkeep[2 * t + 1] = (ok[t][2] ? 0x0000ffffu : 0u) | (ok[t][3] ? 0xffff0000u : 0u);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = t0 + 16 * t + 4 * q4 + e;
            ok[t][e] = tok < je && tok <= last_vis;
          }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = ok[t][e] ? sacc[t][e] * sc : NEG_INF;
          v[t][e] = x;
          mx = fmaxf(mx, x);
        }
      }
      if (row_ok && !is_list) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int tb = t0 + 16 * t + 4 * q4;
          float* dst = lrow + tb;
          if (tb + 4 <= je) {
            *reinterpret_cast<f32x4u*>(dst) = f32x4u{v[t][0], v[t][1], v[t][2], v[t][3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (tb + e < je) dst[e] = v[t][e];
          }
        }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    // the accumulators are rescaled only when some row's maximum grew
    if (__any(m_new > m_run)) {
      const float alpha = (m_new == NEG_INF) ? 1.f : fast_exp2((m_run - m_new) * LOG2E);
      l_run *= alpha;
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) oacc[dd] *= alpha;
      m_run = m_new;
    }
    const float base = (m_run == NEG_INF) ? 0.f : m_run * LOG2E;
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = v[t][e];
        const float ex = (full || x != NEG_INF) ? fast_exp2(fmaf(x, LOG2E, -base)) : 0.f;
        pb[4 * t + e] = (__bf16)ex;
        psum += ex;
      }
    }
    l_run += psum;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      const int c = 2 * dd + (vcol >> 1);
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(Vs + vrow0 * NCH * 16 + 16 * (c ^ vswz<NCH>(vrow0)) + 8 * (vcol & 1)));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(Vs + vrow1 * NCH * 16 + 16 * (c ^ vswz<NCH>(vrow1)) + 8 * (vcol & 1)));
      u32x4v vw = __builtin_bit_cast(
          u32x4v, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0],
                                                              hi[1], hi[2], hi[3]});
      if (is_list) vw &= vkeep;
      const bf16x8 va = __builtin_bit_cast(bf16x8, vw);
      oacc[dd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[dd], 0, 0, 0);
    }
  }

  if (!wave_active) continue;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) continue;
  if (it.nchunk == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)(it.row0 + qi) * Hq + h) * D;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      const uint32_t b0 = f2bf(oacc[dd][0] * inv), b1 = f2bf(oacc[dd][1] * inv);
      const uint32_t b2 = f2bf(oacc[dd][2] * inv), b3 = f2bf(oacc[dd][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dd + 4 * q4) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
    if (q4 == 0)
      p.lse[(int64_t)(it.row0 + qi) * Hq + h] = l_tot > 0.f ? m_run + logf(l_tot) : NEG_INF;
  } else {
    // the chunk's own normalised output, rounded to bf16 like O itself; the
    // merge weighs it by the chunk's share of the row's softmax mass
    const int64_t pr = it.part_row0 + (int64_t)it.split * R + rho;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* po = reinterpret_cast<uint16_t*>(p.part_o) + pr * D;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      const uint32_t b0 = f2bf(oacc[dd][0] * inv), b1 = f2bf(oacc[dd][1] * inv);
      const uint32_t b2 = f2bf(oacc[dd][2] * inv), b3 = f2bf(oacc[dd][3] * inv);
      *reinterpret_cast<uint2*>(po + 16 * dd + 4 * q4) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
    if (q4 == 0) {
      p.part_ml[2 * pr] = m_run;
      p.part_ml[2 * pr + 1] = l_tot;
    }
  }
  }  // KV heads of the item
  if (wave == 0 && lane == 0) *next_item = (int)next;
}

// One attention item on the MFMA path: a verify chunk (positions [begin, end)
// under the causal limit, logits dumped) or a draft chunk (list entries
// [begin, end); an entry outside [0, L) is masked).
template <int D>
__device__ void attn_tile_dma(const AttnParams& p, const Item& it, char* smem, bool is_list,
                              int* next_item, uint32_t wrap) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // slots of the chunk, padded to whole tiles; -1 marks a masked entry
  int32_t* slots = reinterpret_cast<int32_t*>(smem + dma_smem_bytes<D>() +
                                              logit_stage_bytes((int)(blockDim.x >> 6) - 1));
  const int jb = it.begin, je = it.end;
  const int padded = (je - jb + DMA_TT - 1) / DMA_TT * DMA_TT;
  const int32_t* pt = p.page_table + (int64_t)it.r * p.pt_stride;
  if (is_list) {
    // the list of each packed KV head is padded to whole tiles
    const int ng = max(1, it.ng);
    // LIST_SLOT_BATCH entries per thread and round: their list loads, then
    // their page-table loads, each group in flight together
    const int n = ng * padded, nthr = (int)blockDim.x;
    const int32_t* list0 = p.idx_in + it.off;
    for (int b0 = 0; b0 < n; b0 += LIST_SLOT_BATCH * nthr) {
      int32_t pos[LIST_SLOT_BATCH];
#pragma unroll
      for (int u = 0; u < LIST_SLOT_BATCH; ++u) {
        const int x = b0 + u * nthr + tid;
        const int hd = x / padded, j = x - hd * padded;
        pos[u] = (x < n && jb + j < je) ? list0[(int64_t)hd * it.list_len + jb + j] : -1;
      }
      int32_t sl[LIST_SLOT_BATCH];
#pragma unroll
      for (int u = 0; u < LIST_SLOT_BATCH; ++u)
        sl[u] = (pos[u] >= 0 && pos[u] < it.L) ? pt[pos[u]] : -1;
#pragma unroll
      for (int u = 0; u < LIST_SLOT_BATCH; ++u) {
        const int x = b0 + u * nthr + tid;
        if (x < n) slots[x] = sl[u] < 0 ? -1 : (int32_t)clamp_slot(sl[u], p.num_slots);
      }
    }
    if (ng > 1) {  // the G query rows of every packed head, after the slots
      uint4* qst = reinterpret_cast<uint4*>(slots + ng * padded);
      const uint4* qsrc =
          reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                         ((int64_t)it.row0 * p.Hq + it.g * p.G) * D);
      for (int x = tid; x < ng * p.G * D / 8; x += blockDim.x) qst[x] = qsrc[x];
    }
  } else {
    // VERIFY_SLOT_BATCH page-table entries per thread and round, all their
    // loads in flight before the first store: a 2048-position chunk costs one
    // round trip with 256 threads instead of eight.  (The same batching of the
    // draft lists, with the packed query rows, raised the kernel's registers
    // from 171 to 191 and made the Qwen3-14B-shaped step 7% slower.)
    const int nthr = (int)blockDim.x;
    for (int b0 = 0; b0 < padded; b0 += VERIFY_SLOT_BATCH * nthr) {
      int32_t sl[VERIFY_SLOT_BATCH];
#pragma unroll
      for (int u = 0; u < VERIFY_SLOT_BATCH; ++u) sl[u] = pt[min(jb + b0 + u * nthr + tid, je - 1)];
#pragma unroll
      for (int u = 0; u < VERIFY_SLOT_BATCH; ++u) {
        const int j = b0 + u * nthr + tid;
        if (j < padded) slots[j] = (int32_t)clamp_slot(sl[u], p.num_slots);
      }
    }
  }
  __syncthreads();
  if (wave == (int)(blockDim.x >> 6) - 1)
    dma_producer<D>(p, it, smem, slots, lane);
  else if (is_list)
    dma_consumer<D, true>(p, it, smem, slots, wave, lane, next_item, wrap);
  else
    dma_consumer<D, false>(p, it, smem, slots, wave, lane, next_item, wrap);
}

// ==========================================================================
// VALU gather tile: the G query heads of one query row attend to a set of
// positions -- a draft row's list entries [begin, end), or (fp32 verify) the
// positions [begin, end) under a causal limit.  LPR consecutive lanes read one
// K/V row as 16-byte pieces; partial dot products are reduced with lane
// shuffles; each block's softmax statistics go through LDS; P*V accumulates per
// lane and is summed across waves at the end.  Two blocks of rows are in flight
// in registers while a third is processed.
// ==========================================================================
template <int D, typename T, int GM>
__device__ void gather_tile_valu(const AttnParams& p, const Item& it, char* smem, bool is_list,
                                 int qi, int last_vis, float* lrow, int rho0, int Rr) {
  constexpr int E = Piece<T>::E;   // elements per 16-byte piece
  constexpr int LPR = D / E;       // lanes per K/V row
  constexpr int TPT = 4;           // rows per thread per block
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
  const int G = p.G, Hq = p.Hq, Hkv = p.Hkv, g = it.g;
  const int c = tid % LPR, tl = tid / LPR, NTL = nthr / LPR;
  const int TB = NTL * TPT;
  const int nent = it.end - it.begin;
  const int L = it.L;

  int32_t* slots = reinterpret_cast<int32_t*>(smem);
  float* scs = reinterpret_cast<float*>(slots + DRAFT_MAX_CHUNK);  // [GM][TB]
  float* st = scs + GM * TB;                                         // m[GM], l[GM], alpha[GM]
  float* red = st + 3 * GM;                                          // [nwaves][GM][D]

  const int32_t* ptr = p.page_table + (int64_t)it.r * p.pt_stride;
  const int32_t* list = is_list ? p.idx_in + it.off : nullptr;
  for (int t = tid; t < nent; t += nthr) {
    const int pos = is_list ? list[it.begin + t] : it.begin + t;
    int32_t s = -1;
    if (pos >= 0 && pos < L && pos <= last_vis) s = (int32_t)clamp_slot(ptr[pos], p.num_slots);
    slots[t] = s;
  }
  if (tid < GM) {
    st[tid] = NEG_INF;
    st[GM + tid] = 0.f;
  }

  float qv[GM][E];
  const T* qbase = reinterpret_cast<const T*>(p.q) + ((int64_t)(it.row0 + qi) * Hq + g * G) * D;
#pragma unroll
  for (int hh = 0; hh < GM; ++hh) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (hh < G) v = *reinterpret_cast<const uint4*>(qbase + (int64_t)hh * D + c * E);
    Piece<T>::unpack(v, qv[hh]);
  }
  float oacc[GM][E];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int e = 0; e < E; ++e) oacc[hh][e] = 0.f;

  const T* kpool = reinterpret_cast<const T*>(p.k_pool);
  const T* vpool = reinterpret_cast<const T*>(p.v_pool);
  const float sc = p.sm_scale;
  __syncthreads();

  // Unconditional loads (an invalid entry reads pool row 0) keep the blocks in
  // flight; invalid entries are masked when the block is processed.
  auto fetch = [&](int b0, int32_t (&s_)[TPT], uint4 (&k_)[TPT], uint4 (&v_)[TPT]) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = b0 + tl + NTL * i;
      const int32_t sv = slots[min(t, nent - 1)];
      s_[i] = (t < nent) ? sv : -1;
      const int64_t off = ((int64_t)max(sv, 0) * Hkv + g) * D + c * E;
      k_[i] = load_kv16(kpool + off);
      v_[i] = load_kv16(vpool + off);
    }
  };
  auto process = [&](int b0, const int32_t (&sl)[TPT], const uint4 (&kr)[TPT],
                     const uint4 (&vr)[TPT]) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      float kf[E];
      Piece<T>::unpack(kr[i], kf);
      float dot[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaf(qv[hh][e], kf[e], a);
        dot[hh] = group_sum<LPR>(a);
      }
      const int u = tl + NTL * i;
      if (c == 0) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh)
          if (hh < G) scs[hh * TB + u] = (sl[i] >= 0) ? dot[hh] * sc : NEG_INF;
      }
    }
    __syncthreads();
    if (lrow != nullptr) {
      for (int x = tid; x < G * TB; x += nthr) {
        const int hh = x / TB, u = x % TB;
        if (b0 + u < nent) lrow[(int64_t)hh * L + it.begin + b0 + u] = scs[hh * TB + u];
      }
      __syncthreads();  // the loop below rewrites scs in place
    }
    for (int hh = wave; hh < G; hh += nwaves) {
      float mx = NEG_INF;
      for (int u = lane; u < TB; u += 64) mx = fmaxf(mx, scs[hh * TB + u]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = st[hh];
      const float m_new = fmaxf(m_old, mx);
      float alpha = 1.f, base = 0.f;
      if (m_new != NEG_INF) {
        alpha = fast_exp2((m_old - m_new) * LOG2E);
        base = m_new * LOG2E;
      }
      float s = 0.f;
      for (int u = lane; u < TB; u += 64) {
        const float x = scs[hh * TB + u];
        const float e = (x == NEG_INF) ? 0.f : fast_exp2(fmaf(x, LOG2E, -base));
        scs[hh * TB + u] = e;
        s += e;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) {
        st[hh] = m_new;
        st[GM + hh] = st[GM + hh] * alpha + s;
        st[2 * GM + hh] = alpha;
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      if (hh < G) {
        const float a = st[2 * GM + hh];
#pragma unroll
        for (int e = 0; e < E; ++e) oacc[hh][e] *= a;
      }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      if (sl[i] < 0) continue;
      const int u = tl + NTL * i;
      float vf[E];
      Piece<T>::unpack(vr[i], vf);
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        if (hh < G) {
          const float pp = scs[hh * TB + u];
#pragma unroll
          for (int e = 0; e < E; ++e) oacc[hh][e] = fmaf(pp, vf[e], oacc[hh][e]);
        }
      }
    }
    __syncthreads();  // scs and st reused by the next block
  };

  int32_t sA[TPT], sB[TPT];
  uint4 kA[TPT], vA[TPT], kB[TPT], vB[TPT];
  fetch(0, sA, kA, vA);
  if (TB < nent) fetch(TB, sB, kB, vB);
  for (int b0 = 0; b0 < nent; b0 += 2 * TB) {
    process(b0, sA, kA, vA);
    if (b0 + 2 * TB < nent) fetch(b0 + 2 * TB, sA, kA, vA);
    if (b0 + TB >= nent) break;
    process(b0 + TB, sB, kB, vB);
    if (b0 + 3 * TB < nent) fetch(b0 + 3 * TB, sB, kB, vB);
  }

  // lanes of one wave that share c hold partial sums of the same output slice
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
      for (int e = 0; e < E; ++e) oacc[hh][e] += __shfl_xor(oacc[hh][e], off);
  if (lane < LPR) {
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
      if (hh < G)
#pragma unroll
        for (int e = 0; e < E; ++e) red[(wave * GM + hh) * D + c * E + e] = oacc[hh][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += nthr) {
    const int hh = x / D, d = x % D;
    float acc = 0.f;
    for (int w = 0; w < nwaves; ++w) acc += red[(w * GM + hh) * D + d];
    const float m = st[hh], l = st[GM + hh];
    const int h = g * G + hh;
    if (it.nchunk == 1) {
      const int64_t orow = (int64_t)(it.row0 + qi) * Hq + h;
      store_out<T>(reinterpret_cast<T*>(p.o) + orow * D + d, l > 0.f ? acc / l : 0.f);
      if (d == 0) p.lse[orow] = l > 0.f ? m + logf(l) : NEG_INF;
    } else {
      const int64_t pr = it.part_row0 + (int64_t)it.split * Rr + rho0 + hh;
      store_out<T>(reinterpret_cast<T*>(p.part_o) + pr * D + d, l > 0.f ? acc / l : 0.f);
      if (d == 0) {
        p.part_ml[2 * pr] = m;
        p.part_ml[2 * pr + 1] = l;
      }
    }
  }
}


// Runs one item; returns true when it has stored the workgroup's next draw
// at next_item (the MFMA path does so near its end), false when the caller
// must draw.  The result is the same for every thread of the workgroup.
template <int D, typename T, int GM>
__device__ __forceinline__ bool attn_body(const AttnParams& p, int item, char* smem,
                                          int* next_item, uint32_t wrap) {
  const Item it = p.items[item];
  if (it.kind == KIND_NOP) return false;
  if constexpr (sizeof(T) == 2) {
    attn_tile_dma<D>(p, it, smem, it.kind == KIND_DRAFT, next_item, wrap);
    return true;
  } else if (it.kind == KIND_VERIFY) {
    const int qi = it.qi;
    const int last_vis = it.L - (p.k + 1) + qi;
    float* lrow = p.logits + it.off + ((int64_t)qi * p.Hq + it.g * p.G) * it.L;
    gather_tile_valu<D, T, GM>(p, it, smem, false, qi, last_vis, lrow, qi * p.G, (p.k + 1) * p.G);
  } else {
    gather_tile_valu<D, T, GM>(p, it, smem, true, 0, 0x7fffffff, nullptr, 0, p.G);
  }
  return false;
}

// Persistent workgroups: the launch has as many workgroups as fit on the chip
// at once, and each one keeps drawing the next item of the plan (longest
// first) until none is left.  Whichever CU frees first, on any XCD, takes the
// next item, so an XCD that runs slower simply processes fewer items; with
// one workgroup per item, workgroup i always runs on XCD i % 8 and every XCD
// would own a fixed eighth of the work.
// When two workgroups fit per CU, workgroup b starts on item b without a
// draw: all G workgroups drawing from one counter at once queue at that
// address, and the last got its first item about 6 us after the launch began
// (3 us on average, measured on 512 workgroups).  With F such first items
// (min(G, n), or none), the counter hands out draw t = 0, 1, ...: items F,
// F+1, ... while S = n - F of them last, then one past-the-end draw per
// workgroup (index e = t - S).  That is S + G draws, so atomicInc wrapping at
// S + G - 1 hands out every value once and leaves the counter at 0 for the
// next launch that uses it.  A workgroup without a first item (b >= F) draws
// at once.  The draw for the next item lands in the other entry of s_item,
// which every thread finished reading before the previous iteration's closing
// barrier.  (Measured against drawing every item: draft-only Qwen3-8B-shaped
// batches 11-15% faster at s <= 0.05, the mixed Qwen3-1.7B, Qwen3-8B and
// long-context steps 0.6-1.5% faster; the Qwen3-14B-shaped step, one
// workgroup per CU, 1.3% slower, so such launches draw every item.  Mapping
// draws to items in the consumer wave instead of here made both Qwen3 steps
// 5% slower.)
template <int D, typename T, int GM>
__device__ __forceinline__ void attn_loop(const AttnParams& p, char* smem) {
  __shared__ int s_item[2];
  // F workgroups start on their own item (none when the launch draws every
  // item); the counter hands out the S = n - F others, then G past-the-end
  // draws
  const int G = (int)gridDim.x, n = p.n_items, F = p.first_static ? min(G, n) : 0, S = n - F;
  const uint32_t wrap = (uint32_t)(S + G) - 1u;
  const bool static_first = (int)blockIdx.x < F;
  if (!static_first) {
    if (threadIdx.x == 0) s_item[0] = (int)atomicInc(p.ticket, wrap);
    __syncthreads();
  }
  for (int k = 0, first = static_first ? 1 : 0;; k ^= 1, first = 0) {
    const int t = first ? 0 : s_item[k];
    const int item = first ? (int)blockIdx.x : (t < S ? F + t : n + (t - S));
    if (item >= n) {  // the same value for the whole workgroup
      // Out of work.  Every workgroup draws exactly one ticket past the last
      // item; the first half of those draws (workgroups that run out while
      // others still finish their last items) copy the post-pass and selection
      // records from the pinned plan into the workspace, one contiguous run of
      // 16-byte pieces per workgroup and round.  The launches after this one
      // then read their records from device memory instead of across PCIe,
      // where the read is on their critical path.
      const int e = item - n;
      const int nc = max(1, G / 2);
      if (e < nc) {
        for (int c = e * (int)blockDim.x + (int)threadIdx.x; c < p.plan_n16; c += nc * (int)blockDim.x)
          p.plan_dst[c] = p.plan_src[c];
        for (int c = e * (int)blockDim.x + (int)threadIdx.x; c < p.zero_n16; c += nc * (int)blockDim.x)
          p.zero_dst[c] = make_uint4(0u, 0u, 0u, 0u);
      }
      // The last of those draws comes after every other workgroup's: no
      // plan record is read after it.
      if (p.done && e == G - 1 && threadIdx.x == 0)
        __hip_atomic_store(p.done, p.done_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    const bool drew = attn_body<D, T, GM>(p, item, smem, &s_item[k ^ 1], wrap);
    if (!drew && threadIdx.x == 0)
      s_item[k ^ 1] = (int)atomicInc(p.ticket, wrap);
    __syncthreads();  // LDS is free and the next draw is visible
  }
}

// All attention items of a call (or, for a mixed batch with overlap, its
// verify items).
template <int D, typename T, int GM>
__global__ void __launch_bounds__(512) attn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  attn_loop<D, T, GM>(p, smem);
}

// The draft items of a mixed batch, launched on the side stream (same work
// per item; a separate symbol so that profiles tell the two launches apart).
template <int D, typename T, int GM>
__global__ void __launch_bounds__(512) attn_kernel_draft(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  attn_loop<D, T, GM>(p, smem);
}

// ==========================================================================
// PillarAttn post-pass
// ==========================================================================
// split-K merge of rows [j0, j1) of one (r, g): m* = max_s m_s,
// l* = sum_s l_s e^{m_s - m*}, O = sum_s e^{m_s - m*} O_s / l*, LSE = m* + ln l*.
// The (m, l) pairs of every chunk are staged in LDS, one wave per row turns
// them into weights in place (lane s % 64 alone touches pair s), and each
// thread then owns one (row, 4 dims) column of O.
template <int D, typename T>
__device__ void merge_rows(const PostParams& p, const PostItem& it, char* smem) {
  constexpr int D4 = D / 4;
  static_assert(MERGE_ROWS * D4 <= 256, "one O column per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int G = p.G;
  const int R = it.rows_q * G;
  const int ns = it.nchunk;
  const int rho0 = it.j0, nr = it.j1 - it.j0;
  float* w_s = reinterpret_cast<float*>(smem);  // [MERGE_ROWS][ns] (m, l) pairs
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml);
  for (int x = tid; x < nr * ns; x += blockDim.x) {
    const int rr = x / ns, sidx = x % ns;
    const float2 v = ml[it.part_row0 + (int64_t)sidx * R + rho0 + rr];
    w_s[2 * x] = v.x;
    w_s[2 * x + 1] = v.y;
  }
  __syncthreads();
  for (int rr = wave; rr < nr; rr += nwaves) {
    float* pr = w_s + 2 * rr * ns;
    float mx = NEG_INF;
    for (int sidx = lane; sidx < ns; sidx += 64) mx = fmaxf(mx, pr[2 * sidx]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float ls = 0.f;
    if (mx != NEG_INF)
      for (int sidx = lane; sidx < ns; sidx += 64) {
        const float m = pr[2 * sidx];
        if (m != NEG_INF) ls = fmaf(pr[2 * sidx + 1], fast_exp2((m - mx) * LOG2E), ls);
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
    // partials are each chunk's normalised output: weight = its share of the
    // row's softmax mass, l_s e^{m_s - m*} / l*
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    for (int sidx = lane; sidx < ns; sidx += 64) {
      const float m = pr[2 * sidx];
      pr[2 * sidx] = (m == NEG_INF || inv == 0.f) ? 0.f : fast_exp2((m - mx) * LOG2E) * pr[2 * sidx + 1] * inv;
    }
    if (lane == 0) {
      const int rho = rho0 + rr, qi = rho / G, hh = rho % G;
      p.lse[(int64_t)(it.row0 + qi) * p.Hq + it.g * G + hh] = ls > 0.f ? mx + logf(ls) : NEG_INF;
    }
  }
  __syncthreads();
  if (tid >= nr * D4) return;
  const int rr = tid / D4, d4 = tid % D4;
  const int rho = rho0 + rr;
  // partials are stored in the output's type (bf16 or fp32)
  const T* src = reinterpret_cast<const T*>(p.part_o) + (it.part_row0 + rho) * D + 4 * d4;
  const int64_t sstride = (int64_t)R * D;
  const float* w = w_s + 2 * rr * ns;  // weight of chunk s at w[2 s]
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // NB partials per round trip (entries past ns re-read the last partial at
  // weight 0): 16 when there are more than 8, so that 16 chunks take one
  auto merge_in = [&](auto nb) {
    constexpr int NB = decltype(nb)::value;
    for (int s0 = 0; s0 < ns; s0 += NB) {
      float4 o[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) o[u] = load4<T>(src + min(s0 + u, ns - 1) * sstride);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float wu = (s0 + u < ns) ? w[2 * (s0 + u)] : 0.f;
        acc.x = fmaf(wu, o[u].x, acc.x);
        acc.y = fmaf(wu, o[u].y, acc.y);
        acc.z = fmaf(wu, o[u].z, acc.z);
        acc.w = fmaf(wu, o[u].w, acc.w);
      }
    }
  };
  if (ns > 8)
    merge_in(std::integral_constant<int, 16>{});
  else
    merge_in(std::integral_constant<int, 8>{});
  const int qi = rho / G, hh = rho % G;
  const int64_t orow = (int64_t)(it.row0 + qi) * p.Hq + it.g * G + hh;
  T* dst = reinterpret_cast<T*>(p.o) + orow * D + 4 * d4;
  store_out<T>(dst + 0, acc.x);
  store_out<T>(dst + 1, acc.y);
  store_out<T>(dst + 2, acc.z);
  store_out<T>(dst + 3, acc.w);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP only: row_shr
// 1, 2, 4, 8 scans each row of 16 lanes; row_bcast:15 then row_bcast:31 carry
// the row totals into the later rows.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_rows<0x111, 0xf>(v);  // row_shr:1
  v += dpp_rows<0x112, 0xf>(v);  // row_shr:2
  v += dpp_rows<0x114, 0xf>(v);  // row_shr:4
  v += dpp_rows<0x118, 0xf>(v);  // row_shr:8
  v += dpp_rows<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_rows<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Block-wide exclusive prefix of per-thread counts (DPP wave scan + per-wave
// totals in LDS).  Returns the prefix; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    const uint32_t s = wsum[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();  // wsum reusable
  *total = all;
  return before + incl - v;
}

// Sum, AND and OR over each row of 16 lanes (DPP, no LDS); every lane of the
// row receives the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t row_sum_u32(uint32_t v) {
  v += dppu<DPP_XOR1>(v);
  v += dppu<DPP_XOR2>(v);
  v += dppu<DPP_HALF_MIRROR>(v);
  v += dppu<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ uint32_t row_and_u32(uint32_t v) {
  v &= dppu<DPP_XOR1>(v);
  v &= dppu<DPP_XOR2>(v);
  v &= dppu<DPP_HALF_MIRROR>(v);
  v &= dppu<DPP_MIRROR>(v);
  return v;
}
__device__ __forceinline__ uint32_t row_or_u32(uint32_t v) {
  v |= dppu<DPP_XOR1>(v);
  v |= dppu<DPP_XOR2>(v);
  v |= dppu<DPP_HALF_MIRROR>(v);
  v |= dppu<DPP_MIRROR>(v);
  return v;
}

constexpr int SELECT_FINISH = 64;  // candidates ranked directly by one wave
constexpr int SELECT_THREADS = 1024;  // every selection workgroup
constexpr int HIST_PER = HIST_BINS / SELECT_THREADS;  // histogram bins per thread
static_assert(HIST_PER * SELECT_THREADS == HIST_BINS, "bins split evenly");
constexpr int SELECT_BITMAP_BITS = 1 << 18;  // longest row whose selected positions are marked in LDS

// Bits of the selection launch's position bitmap for rows of at most max_len
// scores: none when every row fits the register span.
int select_bitmap_bits(int max_len) {
  if (max_len <= SELECT_SPAN) return 0;
  return std::min((max_len + 31) / 32 * 32, SELECT_BITMAP_BITS);
}
constexpr int SELECT_BATCH = 4;    // chunks loaded per batch when a row is longer than one chunk

// The boundary bin of the K-th largest key from a row's histogram: sv[0] =
// bin << HIST_SHIFT, sv[1] = K minus the keys in higher bins (the K-th key's
// rank inside the bin), sv[2] = the keys in the bin, or 0xffffffff when no bin
// holds the K-th key (inconsistent counts).
__device__ __forceinline__ void hist_boundary(const uint32_t* hist, int K, uint32_t* sv, uint32_t* wsum) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sv[0] = 0u;
    sv[1] = (uint32_t)K;
    sv[2] = 0xffffffffu;
  }
  // thread t holds bins 2047 - HIST_PER t down to 2048 - HIST_PER (t + 1)
  const int b0 = HIST_BINS - 1 - HIST_PER * tid;
  uint32_t hv[HIST_PER];
  uint32_t mine = 0u;
#pragma unroll
  for (int b = 0; b < HIST_PER; ++b) {
    hv[b] = hist[b0 - b];
    mine += hv[b];
  }
  uint32_t tot;
  const uint32_t above = block_exclusive_scan(mine, wsum, &tot);
  if (above < (uint32_t)K && above + mine >= (uint32_t)K) {  // one thread owns the K-th key
    uint32_t acc = above;
#pragma unroll
    for (int b = 0; b < HIST_PER; ++b) {
      if (acc < (uint32_t)K && acc + hv[b] >= (uint32_t)K) {
        sv[0] = (uint32_t)(b0 - b) << HIST_SHIFT;
        sv[1] = (uint32_t)K - acc;
        sv[2] = hv[b];
      }
      acc += hv[b];
    }
  }
  __syncthreads();
}

// Top-K of L non-negative fp32 scores (their bit patterns order like the
// values).  MSB-first radix select with 4-bit digits finds the K-th largest
// value tau and how many positions equal to it are kept; the compaction then
// writes every position above tau and the lowest positions equal to tau,
// ascending.  Thread t owns the KPT consecutive positions c0 + KPT t + [0, KPT)
// of each chunk of KPT*nthr positions; keys stay in registers when L fits one
// chunk and are re-read chunk by chunk otherwise.
//   - The digits every key shares (block-wide AND/OR) are skipped.
//   - A pass counts without atomics: 4-bit counters packed in two registers
//     per thread (KPT <= 8 per chunk), widened to bytes and summed over rows
//     of 16 lanes with DPP (<= 128 per byte), then to 32 bits per digit.
//   - Once the bucket holding the K-th key has at most 64 keys, they are
//     gathered into LDS and one wave ranks them directly.
//   - hist, when given, holds the row's keys counted by bits 30..20 (2048
//     bins; the sign bit of a non-negative score is 0), summed by the
//     launch that wrote the scores.  The bin of the K-th largest key then
//     fixes those bits at once, replacing the AND/OR walk and three passes
//     (each a block-wide round, and on rows of many chunks a re-read).
template <int KPT>
__device__ __forceinline__ void select_topk(const float* scores, int L, int K, int32_t* out, char* smem,
                                            const uint32_t* hist = nullptr, uint32_t* bm = nullptr,
                                            int32_t* cpos = nullptr, int bm_bits = 0) {
  static_assert(KPT % 4 == 0 && KPT <= 8, "keys are loaded four at a time; nibble counters");
  uint32_t* sv = reinterpret_cast<uint32_t*>(smem);  // prefix, rem, bucket count, gathered, and/or
  uint32_t* wsum = sv + 8;                           // [16] block scans
  uint32_t* tab = wsum + 16;                         // [waves * 4 rows][16 digits]
  uint32_t* ckey = tab + 16 * 64;                    // [SELECT_FINISH] candidate keys
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(scores);
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int nrows = (nthr >> 6) * 4;
  const int span = KPT * nthr;
  const bool resident = L <= span;
  uint32_t key[KPT];
  // Every load of a batch is issued before any of them is used, at an address
  // clamped to the quad holding position L-1, and positions at or past L are
  // set to key 0 only afterwards.  A per-thread branch between two loads makes
  // the compiler wait for the first before issuing the second (a batch was one
  // round trip per load), and a scalar fallback path for unaligned rows was
  // merged with this one into 4-byte loads.  The row starts 16-byte aligned and
  // its storage extends to L rounded up to a multiple of 4 (both callers' rows
  // are workspace rows laid out so), so that quad is read whole.
  const int jq = (L - 1) & ~3;
  auto load_raw = [&](uint32_t (&dst)[KPT], int c0) {
    const int j0 = c0 + KPT * tid;
#pragma unroll
    for (int m = 0; m < KPT; m += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(keys + min(j0 + m, jq));
      dst[m] = v.x;
      dst[m + 1] = v.y;
      dst[m + 2] = v.z;
      dst[m + 3] = v.w;
    }
  };
  auto mask_past_end = [&](uint32_t (&dst)[KPT], int c0) {
    const int j0 = c0 + KPT * tid;
#pragma unroll
    for (int m = 0; m < KPT; ++m)
      if (j0 + m >= L) dst[m] = 0u;
  };
  // Calls body(c0) for every chunk with its keys in key[].  Rows longer than
  // one chunk are re-read on every walk, SELECT_BATCH chunks per batch of loads
  // so that a walk costs one round trip per batch, not per chunk.
  auto each_chunk = [&](auto&& body) {
    if (resident) {
      body(0);
      return;
    }
    for (int c0 = 0; c0 < L; c0 += SELECT_BATCH * span) {
      uint32_t kb[SELECT_BATCH][KPT];
#pragma unroll
      for (int q = 0; q < SELECT_BATCH; ++q) load_raw(kb[q], c0 + q * span);
#pragma unroll
      for (int q = 0; q < SELECT_BATCH; ++q) {
        if (c0 + q * span < L) {  // the same for every thread
#pragma unroll
          for (int m = 0; m < KPT; ++m) key[m] = kb[q][m];
          mask_past_end(key, c0 + q * span);
          body(c0 + q * span);
        }
      }
    }
  };
  if (resident) {
    load_raw(key, 0);
    mask_past_end(key, 0);
  }
  int shift;
  uint32_t mask;
  if (hist) {
    // the bin of the K-th key fixes bits 30..20 (a bin count of 0xffffffff,
    // when no bin holds it, sends the walk through every digit below)
    hist_boundary(hist, K, sv, wsum);
    shift = HIST_SHIFT - 4;
    mask = 0xffffffffu << HIST_SHIFT;
  } else {
    // bits shared by every key: AND and OR over the block
    if (tid == 0) {
      sv[4] = 0xffffffffu;
      sv[5] = 0u;
    }
    __syncthreads();
    {
      uint32_t va = 0xffffffffu, vo = 0u;
      each_chunk([&](int c0) {
        const int j0 = c0 + KPT * tid;
#pragma unroll
        for (int m = 0; m < KPT; ++m)
          if (j0 + m < L) {
            va &= key[m];
            vo |= key[m];
          }
      });
      va = row_and_u32(va);
      vo = row_or_u32(vo);
      if ((lane & 15) == 0) {
        atomicAnd(&sv[4], va);
        atomicOr(&sv[5], vo);
      }
    }
    if (tid == 0) {
      sv[0] = 0u;
      sv[1] = (uint32_t)K;
    }
    __syncthreads();
    const uint32_t diff = sv[4] ^ sv[5];
    shift = diff == 0u ? 0 : (31 - __builtin_clz(diff)) / 4 * 4;  // top differing digit
    mask = shift >= 28 ? 0u : 0xffffffffu << (shift + 4);
    if (tid == 0) sv[0] = sv[4] & mask;  // the shared leading digits
    __syncthreads();
  }
  // a histogram bin small enough already goes straight to the direct ranking
  bool finish = hist != nullptr && sv[2] <= (uint32_t)SELECT_FINISH;
  for (; shift >= 0 && !finish; shift -= 4) {
    const uint32_t prefix = sv[0];
    uint32_t acc[16];  // per row of 16 lanes
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = 0u;
    each_chunk([&](int c0) {
      (void)c0;
      // Positions past L hold key 0, the smallest value, and come after every
      // real position in the tie order, so counting them never moves the
      // K-th largest real key (K <= L); the compaction skips them.
      uint32_t lo = 0u, hi = 0u;  // nibble counters of digits 0..7 and 8..15
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const bool inb = (key[m] & mask) == prefix;
        const uint32_t d = (key[m] >> shift) & 15u;
        const uint32_t inc = inb ? (1u << (4u * (d & 7u))) : 0u;
        if (d < 8u)
          lo += inc;
        else
          hi += inc;
      }
      // bytes of w: digits (0,2,4,6), (1,3,5,7), (8,10,12,14), (9,11,13,15)
      const uint32_t w[4] = {row_sum_u32(lo & 0x0f0f0f0fu), row_sum_u32((lo >> 4) & 0x0f0f0f0fu),
                             row_sum_u32(hi & 0x0f0f0f0fu), row_sum_u32((hi >> 4) & 0x0f0f0f0fu)};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[8 * (q >> 1) + 2 * e + (q & 1)] += (w[q] >> (8 * e)) & 255u;
    });
    if ((lane & 15) == 0) {
      uint32_t* row = tab + 16 * (wave * 4 + (lane >> 4));
#pragma unroll
      for (int d = 0; d < 16; d += 4)
        *reinterpret_cast<uint4*>(row + d) = make_uint4(acc[d], acc[d + 1], acc[d + 2], acc[d + 3]);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l: digit dl = 15 - (l & 15) over rows (l >> 4) + 4 i
      const int dl = 15 - (lane & 15);
      uint32_t cnt = 0u;
#pragma unroll 4
      for (int r = lane >> 4; r < nrows; r += 4) cnt += tab[16 * r + dl];
      cnt += __shfl_xor(cnt, 16);
      cnt += __shfl_xor(cnt, 32);
      uint32_t incl = cnt;  // inclusive scan inside each row of 16 lanes
      incl += dpp_rows<0x111, 0xf>(incl);
      incl += dpp_rows<0x112, 0xf>(incl);
      incl += dpp_rows<0x114, 0xf>(incl);
      incl += dpp_rows<0x118, 0xf>(incl);
      const uint32_t rem = sv[1];
      const uint32_t excl = incl - cnt;
      if (lane < 16 && excl < rem && incl >= rem) {
        sv[0] = prefix | ((uint32_t)dl << shift);
        sv[1] = rem - excl;
        sv[2] = cnt;
      }
    }
    mask |= 15u << shift;
    __syncthreads();
    if (sv[2] <= (uint32_t)SELECT_FINISH && shift > 0) {
      finish = true;
      break;
    }
  }
  // A row longer than the register span, with a position bitmap in LDS: the
  // gather of the final bucket also marks every position above the bucket,
  // the ranking marks the bucket's chosen positions, and the list is written
  // from the bitmap instead of from a second pass over the row.
  const bool use_bm = finish && bm != nullptr && cpos != nullptr && !resident && L <= bm_bits;
  if (finish) {
    // gather the keys of the chosen bucket (in any order: only their values
    // are ranked) through an LDS counter, so the walk needs no block scans,
    // and rank them in one wave
    const uint32_t prefix = sv[0];
    if (tid == 0) sv[3] = 0u;
    if (use_bm)
      for (int w = tid; w < (L + 31) >> 5; w += nthr) bm[w] = 0u;
    __syncthreads();
    if (use_bm) {
      each_chunk([&](int c0) {
        const int j0 = c0 + KPT * tid;  // a multiple of 8: the thread's positions share one bitmap word
        uint32_t above = 0u;
#pragma unroll
        for (int m = 0; m < KPT; ++m)
          if (j0 + m < L) {
            const uint32_t hk = key[m] & mask;
            if (hk == prefix) {
              const uint32_t pos = atomicAdd(&sv[3], 1u);
              if (pos < (uint32_t)SELECT_FINISH) {
                ckey[pos] = key[m];
                cpos[pos] = j0 + m;
              }
            } else if (hk > prefix) {
              above |= 1u << ((j0 + m) & 31);
            }
          }
        if (above != 0u) atomicOr(&bm[j0 >> 5], above);
      });
    } else {
      each_chunk([&](int c0) {
        const int j0 = c0 + KPT * tid;
#pragma unroll
        for (int m = 0; m < KPT; ++m)
          if (j0 + m < L && (key[m] & mask) == prefix) {
            const uint32_t pos = atomicAdd(&sv[3], 1u);
            if (pos < (uint32_t)SELECT_FINISH) ckey[pos] = key[m];
          }
      });
    }
    __syncthreads();
    if (wave == 0) {
      const int nc = (int)sv[2];
      const uint32_t rem = sv[1];
      const uint32_t mine = lane < nc ? ckey[lane] : 0u;
      uint32_t gt = 0u, eq = 0u;
      for (int j = 0; j < nc; ++j) {  // candidate j broadcast from its lane
        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
        gt += o > mine ? 1u : 0u;
        eq += o == mine ? 1u : 0u;
      }
      if (lane < nc && gt < rem && gt + eq >= rem) {
        sv[0] = mine;
        sv[1] = rem - gt;
      }
    }
    __syncthreads();
    if (use_bm) {
      if (wave == 0) {
        // the bucket's keys above the K-th, and its equal keys in position
        // order until the remaining count is taken
        const int nc = min((int)sv[2], min((int)sv[3], SELECT_FINISH));
        const uint32_t tau = sv[0], req = sv[1];
        const uint32_t mine = lane < nc ? ckey[lane] : 0u;
        const int mpos = lane < nc ? cpos[lane] : 0;
        uint32_t before = 0u;
        for (int j = 0; j < nc; ++j) {
          const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
          const int op = __builtin_amdgcn_readlane(mpos, j);
          before += (o == tau && op < mpos) ? 1u : 0u;
        }
        const bool take = lane < nc && (mine > tau || (mine == tau && before < req));
        if (take && mpos >= 0 && mpos < L) atomicOr(&bm[mpos >> 5], 1u << (mpos & 31));
      }
      __syncthreads();
      const int words = (L + 31) >> 5;
      const int wpt = (words + nthr - 1) / nthr;
      const int w0 = tid * wpt, w1 = min(w0 + wpt, words);
      uint32_t cnt = 0u;
      for (int w = w0; w < w1; ++w) cnt += (uint32_t)__popc(bm[w]);
      uint32_t tot;
      uint32_t pos = block_exclusive_scan(cnt, wsum, &tot);
      for (int w = w0; w < w1; ++w) {
        uint32_t b = bm[w];
        while (b != 0u) {
          const int t = __builtin_ctz(b);
          b &= b - 1u;
          if (pos < (uint32_t)K) out[pos++] = (w << 5) + t;
        }
      }
      return;
    }
  }
  const uint32_t tau = sv[0], rem = sv[1];
  uint32_t base_eq = 0, base_gt = 0;
  each_chunk([&](int c0) {
    const int j0 = c0 + KPT * tid;
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const bool ok = j0 + m < L;
      n_gt += (ok && key[m] > tau) ? 1u : 0u;
      n_eq += (ok && key[m] == tau) ? 1u : 0u;
    }
    // one scan of both counts (each below 2^16 within a chunk)
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan(n_gt | (n_eq << 16), wsum, &tot);
    const uint32_t gt_before = base_gt + (pre & 0xffffu);
    const uint32_t eq_before = base_eq + (pre >> 16);
    // equal keys are kept in position order until rem of them are taken
    const uint32_t eq_keep = eq_before >= rem ? 0u : min(n_eq, rem - eq_before);
    uint32_t pos = gt_before + min(eq_before, rem);
    uint32_t eq_seen = 0;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const bool ok = j0 + m < L;
      bool take = ok && key[m] > tau;
      if (ok && key[m] == tau) {
        take = eq_seen < eq_keep;
        ++eq_seen;
      }
      if (take && pos < (uint32_t)K) out[pos++] = j0 + m;
    }
    base_gt += tot & 0xffffu;
    base_eq += tot >> 16;
  });
}

// Four logits of an averaged row.  A row starts 16-byte aligned only when L
// and the request's logits offset are multiples of 4, so the load type asks for
// 4-byte alignment (gfx950 serves 16-byte global loads at any 4-byte
// boundary).  The attention launch wrote these logits just before: when all of
// the step's logits fit the Infinity Cache, plain loads find them there;
// otherwise the streaming hint (each logit is read once) is faster.
template <bool CACHED>
__device__ __forceinline__ f32x4u load_logits4(const float* src) {
  if constexpr (CACHED)
    return *reinterpret_cast<const f32x4u*>(src);
  else
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4u*>(src));
}
template <bool CACHED>
__device__ __forceinline__ float load_logit(const float* src) {
  if constexpr (CACHED)
    return *src;
  else
    return __builtin_nontemporal_load(src);
}

constexpr int POST_THREADS = 256;
constexpr int AVG_PREFETCH = 12;  // averaged terms whose logits load before the LSE rebuild (of 4-16)

// Dynamic LDS of an averaging item: the LSE (4 B) and logits row offset (8 B)
// of every averaged term, then the row's 2048-bin score histogram.
__host__ __device__ constexpr size_t post_hist_offset(int terms) {
  return ((size_t)(terms * 4 + 7) / 8 * 8 + (size_t)terms * 8 + 15) / 16 * 16;
}
static_assert(AVG_SPAN == 4 * POST_THREADS, "an averaging thread owns four positions");

template <int D, typename T, bool CACHED>
__global__ void __launch_bounds__(POST_THREADS) post_kernel(PostParams p) {
  // merge: (m, l) pairs then weights of MERGE_ROWS rows; averaging: LSE and
  // logits row offsets of the averaged terms
  // dynamic LDS (post_smem_bytes): the (m, l) pairs of MERGE_ROWS rows, or the
  // LSE and logits row offset of every averaged term
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (p.done && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(p.done, p.done_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < p.plan_n16; c += gridDim.x * blockDim.x)
    p.plan_dst[c] = p.plan_src[c];
  const PostItem it = p.items[blockIdx.x];
  if (it.kind == POST_NOP) return;
  if (it.kind == POST_MERGE) {
    merge_rows<D, T>(p, it, smem);
    return;
  }
  // POST_AVG: LSE of the averaged rows (one thread per (row, head)), then
  // their exact scores averaged over positions [j0, j1); each thread owns four
  // consecutive positions (AVG_SPAN = 4 * blockDim.x)
  const int tid = threadIdx.x;
  const int G = p.G, Hq = p.Hq, a = p.avg_row_begin, n = p.avg_row_count;
  const int terms = n * G;
  const int R = it.rows_q * G;
  const int L = it.L;
  float* lse2_s = reinterpret_cast<float*>(smem);
  int64_t* rowoff_s = reinterpret_cast<int64_t*>(smem + (terms * 4 + 7) / 8 * 8);
  const float* lg = p.logits + it.logits_off;
  const int j4 = it.j0 + 4 * tid;
  const int ne = max(0, min(4, it.j1 - j4));  // positions of this thread
  // The logits of the first AVG_PREFETCH terms do not depend on the LSE: they
  // are requested before it is rebuilt, so that their round trip overlaps the
  // one of the (m, l) partials.
  f32x4u pre[AVG_PREFETCH];
  if (ne == 4) {
#pragma unroll
    for (int x = 0; x < AVG_PREFETCH; ++x)
      if (x < terms) {
        const int i = a + x / G, hh = x % G;
        pre[x] = load_logits4<CACHED>(lg + ((int64_t)i * Hq + it.g * G + hh) * L + j4);
      }
  }
  if (it.nchunk == 1) {
    for (int x = tid; x < terms; x += blockDim.x) {
      const int i = a + x / G, hh = x % G;
      lse2_s[x] = p.lse[(int64_t)(it.row0 + i) * Hq + it.g * G + hh] * LOG2E;
      rowoff_s[x] = ((int64_t)i * Hq + it.g * G + hh) * L;
    }
  } else {
    // A group of tpt threads (a power of two within one wave) per term: each
    // combines up to 8 chunks' (m, l) per batch of loads, running max with the
    // sum rescaled as it grows, then the group merges its partial pairs with
    // lane shuffles.  One round trip for up to 8 tpt chunks.
    int tpt = 1;
    while (tpt < 64 && tpt * 2 * terms <= (int)blockDim.x) tpt *= 2;
    const int sub = tid & (tpt - 1), ngrp = (int)blockDim.x / tpt;
    const int ns = it.nchunk;
    for (int x0 = 0; x0 < terms; x0 += ngrp) {  // the same trip count in every lane
      const int x = x0 + tid / tpt;
      const bool live = x < terms;
      const int i = a + (live ? x : 0) / G, hh = (live ? x : 0) % G;
      const int rho = i * G + hh;
      float mstar = NEG_INF, lsum = 0.f;
      if (live)
        for (int s0 = sub; s0 < ns; s0 += 8 * tpt) {
          float mm[8], ll[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int s = min(s0 + u * tpt, ns - 1);
            const int64_t pr = it.part_row0 + (int64_t)s * R + rho;
            const float2 ml = reinterpret_cast<const float2*>(p.part_ml)[pr];  // (m, l) pair
            mm[u] = ml.x;
            ll[u] = ml.y;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (s0 + u * tpt >= ns || mm[u] == NEG_INF) continue;
            if (mm[u] > mstar) {
              lsum = (mstar == NEG_INF) ? 0.f : lsum * fast_exp2((mstar - mm[u]) * LOG2E);
              mstar = mm[u];
            }
            lsum = fmaf(ll[u], fast_exp2((mm[u] - mstar) * LOG2E), lsum);
          }
        }
      for (int off = 1; off < tpt; off <<= 1) {
        const float m2 = __shfl_xor(mstar, off), l2 = __shfl_xor(lsum, off);
        const float mx = fmaxf(mstar, m2);
        if (mx != NEG_INF) {
          lsum = (mstar == NEG_INF ? 0.f : lsum * fast_exp2((mstar - mx) * LOG2E)) +
                 (m2 == NEG_INF ? 0.f : l2 * fast_exp2((m2 - mx) * LOG2E));
          mstar = mx;
        }
      }
      if (live && sub == 0) {
        const float lse = lsum > 0.f ? mstar + logf(lsum) : NEG_INF;
        lse2_s[x] = lse * LOG2E;
        rowoff_s[x] = ((int64_t)i * Hq + it.g * G + hh) * L;
      }
    }
  }
  // The scores are also counted by bits 30..20 into the row's histogram:
  // in LDS here, then added to the row's global counts.
  const bool keep_hist = p.hist != nullptr && it.hist_slot >= 0;
  uint32_t* hist_s = reinterpret_cast<uint32_t*>(smem + post_hist_offset(terms));
  if (keep_hist)
    for (int b = tid; b < HIST_BINS; b += blockDim.x) hist_s[b] = 0u;
  __syncthreads();
  float* pbar = p.pbar + it.pbar_off;
  const float inv = 1.f / (float)terms;
  float res[4] = {0.f, 0.f, 0.f, 0.f};
  if (ne == 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < AVG_PREFETCH; ++x)
      if (x < terms) {
        const float l2 = lse2_s[x];
        const float vv[4] = {pre[x].x, pre[x].y, pre[x].z, pre[x].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[e] += (vv[e] == NEG_INF || l2 == NEG_INF) ? 0.f : fast_exp2(fmaf(vv[e], LOG2E, -l2));
      }
#pragma unroll 16
    for (int x = AVG_PREFETCH; x < terms; ++x) {
      const f32x4u v4 = load_logits4<CACHED>(lg + rowoff_s[x] + j4);
      const float4 v = make_float4(v4.x, v4.y, v4.z, v4.w);
      const float l2 = lse2_s[x];
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] += (vv[e] == NEG_INF || l2 == NEG_INF) ? 0.f : fast_exp2(fmaf(vv[e], LOG2E, -l2));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = acc[e] * inv;
    *reinterpret_cast<float4*>(pbar + j4) = make_float4(res[0], res[1], res[2], res[3]);
  } else if (ne > 0) {
    // The item's last, partial group of positions: the same loop with four
    // 4-byte loads per term.  Positions past j1 re-read the last valid one
    // and are not stored.
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int x = 0; x < terms; ++x) {
      const float* row = lg + rowoff_s[x] + j4;
      float vv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = load_logit<CACHED>(row + min(e, ne - 1));
      const float l2 = lse2_s[x];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] += (vv[e] == NEG_INF || l2 == NEG_INF) ? 0.f : fast_exp2(fmaf(vv[e], LOG2E, -l2));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = acc[e] * inv;
    for (int e = 0; e < ne; ++e) pbar[j4 + e] = res[e];
  }
  if (keep_hist) {
    // the selection orders keys as unsigned bit patterns; a score is >= +0,
    // so its sign bit is 0 (a pattern with it set is not counted: no bin of
    // the selection's search can hold it)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = __float_as_uint(res[e]);
      if (e < ne && key < 0x80000000u) atomicAdd(&hist_s[key >> HIST_SHIFT], 1u);
    }
    __syncthreads();
    uint32_t* hist_g = p.hist + (int64_t)it.hist_slot * HIST_BINS;
    for (int b = tid; b < HIST_BINS; b += blockDim.x) {
      const uint32_t c = hist_s[b];
      if (c) atomicAdd(&hist_g[b], c);
    }
  }
}

// Selection launch: one workgroup per verify (request, KV head).
constexpr int SELECT_KPT = 8;  // keys per thread kept in registers (8192 at 1024 threads)
static_assert(SELECT_THREADS * SELECT_KPT == SELECT_SPAN, "scores kept in registers");

// ---- long rows, one workgroup per SELECT_SPAN-score chunk --------------------
// The SELECT_KPT consecutive keys of thread t in the chunk starting at c0,
// their loads in flight together; positions at or past L read as key 0.  The
// row starts 16-byte aligned and its storage extends to L rounded up to a
// multiple of 4.
__device__ __forceinline__ void chunk_keys(const float* scores, int L, int c0, uint32_t (&key)[SELECT_KPT]) {
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(scores);
  const int j0 = c0 + SELECT_KPT * (int)threadIdx.x, jq = (L - 1) & ~3;
#pragma unroll
  for (int m = 0; m < SELECT_KPT; m += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(keys + min(j0 + m, jq));
    key[m] = v.x;
    key[m + 1] = v.y;
    key[m + 2] = v.z;
    key[m + 3] = v.w;
  }
#pragma unroll
  for (int m = 0; m < SELECT_KPT; ++m)
    if (j0 + m >= L) key[m] = 0u;
}

// Count launch: chunk record blockIdx.x counts its keys above the boundary
// bin and in it, and stores the bin's keys (with their positions) in its own
// candidate region; chunk 0 also records the boundary for the selection
// launch.
__global__ void __launch_bounds__(SELECT_THREADS) select_count_kernel(SelectParams sp) {
  __shared__ uint32_t sv[8];
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, rec = (int)blockIdx.x, lane = tid & 63, wave = tid >> 6;
  const SelChunk c = sp.chunks[rec];
  const int c0 = c.chunk * SELECT_SPAN;
  uint32_t key[SELECT_KPT];
  chunk_keys(sp.pbar + c.pbar_off, c.L, c0, key);  // in flight with the histogram's loads
  if (tid == 0) sv[3] = 0u;  // candidates appended (published by the boundary's barriers)
  hist_boundary(sp.hist + (int64_t)c.hist_slot * HIST_BINS, c.K, sv, wsum);
  const uint32_t bin = sv[0] >> HIST_SHIFT;
  const bool ok = sv[2] != 0xffffffffu;
  if (c.chunk == 0 && tid < 3) sp.row_info[(int64_t)c.hist_slot * 4 + tid] = sv[tid];
  const int j0 = c0 + SELECT_KPT * tid;
  uint32_t n_above = 0u, n_bin = 0u;
#pragma unroll
  for (int m = 0; m < SELECT_KPT; ++m)
    if (j0 + m < c.L) {
      const uint32_t b = key[m] >> HIST_SHIFT;
      n_above += b > bin ? 1u : 0u;
      n_bin += b == bin ? 1u : 0u;
    }
  // the bin's keys go to the chunk's region in any order (their ranking
  // does not depend on it), through an LDS counter
  if (ok && n_bin != 0u) {
    uint32_t* ck = sp.cand_key + (int64_t)rec * SEL_CAND_CAP;
    int32_t* cp = sp.cand_pos + (int64_t)rec * SEL_CAND_CAP;
#pragma unroll
    for (int m = 0; m < SELECT_KPT; ++m)
      if (j0 + m < c.L && (key[m] >> HIST_SHIFT) == bin) {
        const uint32_t pos = atomicAdd(&sv[3], 1u);
        if (pos < (uint32_t)SEL_CAND_CAP) {
          ck[pos] = key[m];
          cp[pos] = j0 + m;
        }
      }
  }
  // both counts summed over the block in one word (each at most SELECT_SPAN)
  const uint32_t wtot = wave_incl_scan(n_above | (n_bin << 16));
  if (lane == 63) wsum[wave] = wtot;
  __syncthreads();
  if (tid == 0) {
    uint32_t tot = 0u;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += wsum[w];
    sp.cnt_above[rec] = tot & 0xffffu;
    sp.cnt_bin[rec] = tot >> 16;
  }
}

// Selection launch, chunk record `rec` of a long row: the row's candidates
// (every chunk's region, gathered into LDS) give the K-th key tau and how many
// keys equal to it are kept (lowest positions first); the chunk's positions
// above tau, and its share of those equal to it, go to the list at the offset
// the earlier chunks leave.
__device__ __forceinline__ void select_chunk(const SelectParams& sp, int rec, char* smem, char* dyn) {
  uint32_t* sv = reinterpret_cast<uint32_t*>(smem);
  uint32_t* wsum = sv + 8;
  uint32_t* cnt16 = wsum + 16;
  // dynamic LDS: the row's candidate keys and positions
  uint32_t* ck = reinterpret_cast<uint32_t*>(dyn);
  int32_t* cp = reinterpret_cast<int32_t*>(dyn + SEL_CAND_CAP * 4);
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const SelChunk c = sp.chunks[rec];
  const float* scores = sp.pbar + c.pbar_off;
  int32_t* out = sp.idx_out + c.idx_off;
  const int c0 = c.chunk * SELECT_SPAN;
  uint32_t key[SELECT_KPT];
  chunk_keys(scores, c.L, c0, key);  // in flight while the candidates are ranked
  const uint32_t* ri = sp.row_info + (int64_t)c.hist_slot * 4;
  uint32_t prefix = ri[0], rem = ri[1];
  const uint32_t hcnt = ri[2];
  // The row's chunk counts (at most 64 chunks: lane l of every wave holds
  // chunk l's) give each chunk's candidate offset, the row's candidate count
  // nc and the keys above the bin in earlier chunks, without block barriers.
  const uint32_t cbv = lane < c.n ? sp.cnt_bin[c.first + lane] : 0u;
  const uint32_t ca = lane < c.chunk ? sp.cnt_above[c.first + lane] : 0u;
  const uint32_t incl = wave_incl_scan(cbv);
  const uint32_t offv = incl - cbv;
  const uint32_t nc = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t above_b = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ca), 63);
  if (hcnt == 0xffffffffu || nc != hcnt || nc > (uint32_t)SEL_CAND_CAP) {
    // too many keys in the boundary bin (or counts that disagree): the row's
    // first chunk selects the whole row alone, by the full radix walk
    if (c.chunk == 0) select_topk<SELECT_KPT>(scores, c.L, c.K, out, smem);
    return;
  }
  // gather: wave w copies the regions of chunks w, w + 16, ...
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  for (int ci = wv; ci < c.n; ci += nthr >> 6) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)offv, ci);
    const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)cbv, ci);
    const uint32_t* gk = sp.cand_key + (int64_t)(c.first + ci) * SEL_CAND_CAP;
    const int32_t* gp = sp.cand_pos + (int64_t)(c.first + ci) * SEL_CAND_CAP;
    for (uint32_t i = lane; i < n; i += 64) {
      ck[o + i] = gk[i];
      cp[o + i] = gp[i];
    }
  }
  __syncthreads();
  if (nc <= 64u) {
    // one wave ranks the candidates directly
    if (wave == 0) {
      if (lane == 0) {  // stands only if no lane holds the K-th key (inconsistent input)
        sv[3] = 0xffffffffu;
        sv[4] = 0u;
        sv[5] = 0u;
      }
      const uint32_t mk = lane < (int)nc ? ck[lane] : 0u;
      const int mp = lane < (int)nc ? cp[lane] : 0x7fffffff;
      uint32_t gt = 0u, eq = 0u;
      for (int j = 0; j < (int)nc; ++j) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
        gt += o > mk ? 1u : 0u;
        eq += o == mk ? 1u : 0u;
      }
      // lanes holding the K-th key (equal keys agree on all three values)
      if (lane < (int)nc && gt < rem && gt + eq >= rem) {
        sv[3] = eq;
        sv[4] = mk;
        sv[5] = rem - gt;
      }
      __builtin_amdgcn_wave_barrier();
      const uint32_t tau = sv[4];
      const uint64_t gt_b = __ballot(lane < (int)nc && mp < c0 && mk > tau);
      const uint64_t eq_b = __ballot(lane < (int)nc && mp < c0 && mk == tau);
      if (lane == 0) {
        sv[6] = (uint32_t)__popcll(gt_b);
        sv[7] = (uint32_t)__popcll(eq_b);
      }
    }
    __syncthreads();
  } else {
    // 4-bit digits below the bin, counted in LDS over the gathered candidates
    uint32_t mask = 0xffffffffu << HIST_SHIFT;
    for (int shift = HIST_SHIFT - 4; shift >= 0; shift -= 4) {
      if (tid < 16) cnt16[tid] = 0u;
      __syncthreads();
      for (int i = tid; i < (int)nc; i += nthr)
        if ((ck[i] & mask) == prefix) atomicAdd(&cnt16[(ck[i] >> shift) & 15u], 1u);
      __syncthreads();
      if (tid == 0) {
        uint32_t acc = 0u;
        sv[3] = 0xffffffffu;  // stands only if no digit holds the K-th key
        for (int d = 15; d >= 0; --d) {
          const uint32_t n = cnt16[d];
          if (acc + n >= rem) {
            sv[3] = n;  // after the last digit: the row's keys equal to tau
            sv[4] = prefix | ((uint32_t)d << shift);
            sv[5] = rem - acc;
            break;
          }
          acc += n;
        }
      }
      __syncthreads();
      prefix = sv[4];
      rem = sv[5];
      mask |= 15u << shift;
      __syncthreads();  // sv[4], sv[5] and cnt16 are rewritten next round
    }
    const uint32_t tau = sv[4];
    uint32_t gt_m = 0u, eq_m = 0u;
    for (int i = tid; i < (int)nc; i += nthr)
      if (cp[i] < c0) {
        gt_m += ck[i] > tau ? 1u : 0u;
        eq_m += ck[i] == tau ? 1u : 0u;
      }
    uint32_t tot;
    (void)block_exclusive_scan(gt_m | (eq_m << 16), wsum, &tot);  // each count below 2^16
    if (tid == 0) {
      sv[6] = tot & 0xffffu;
      sv[7] = tot >> 16;
    }
    __syncthreads();
  }
  const uint32_t tau = sv[4], eq_take = sv[5], gt_b = sv[6], eq_b = sv[7], eq_all = sv[3];
  const uint32_t base = above_b + gt_b + min(eq_b, eq_take);
  const uint32_t quota = eq_take > eq_b ? eq_take - eq_b : 0u;
  const int j0 = c0 + SELECT_KPT * tid;
  // equal keys before this thread's; not needed when the row keeps all of them
  uint32_t eq_rank = 0u;
  if (eq_take < eq_all) {
    uint32_t n_eq = 0u;
#pragma unroll
    for (int m = 0; m < SELECT_KPT; ++m) n_eq += (j0 + m < c.L && key[m] == tau) ? 1u : 0u;
    uint32_t te;
    eq_rank = block_exclusive_scan(n_eq, wsum, &te);
  }
  bool take[SELECT_KPT];
  uint32_t n_take = 0u;
#pragma unroll
  for (int m = 0; m < SELECT_KPT; ++m) {
    const bool in = j0 + m < c.L;
    bool t = in && key[m] > tau;
    if (in && key[m] == tau) {
      t = eq_rank < quota;
      ++eq_rank;
    }
    take[m] = t;
    n_take += t ? 1u : 0u;
  }
  uint32_t tt;
  uint32_t pos = base + block_exclusive_scan(n_take, wsum, &tt);
#pragma unroll
  for (int m = 0; m < SELECT_KPT; ++m)
    if (take[m]) {
      if (pos < (uint32_t)c.K) out[pos] = j0 + m;
      ++pos;
    }
}

// Chunk launch: one workgroup per chunk record (a separate kernel, so that the
// per-row launch keeps its own code: sharing one kernel cost the Qwen3-8B-shaped
// selection 0.7 us).
__global__ void __launch_bounds__(SELECT_THREADS) select_chunk_kernel(SelectParams sp) {
  __shared__ __attribute__((aligned(16))) char smem[(24 + 16 * 64 + SELECT_FINISH) * 4];
  extern __shared__ __attribute__((aligned(16))) char dyn[];  // the row's candidate keys and positions
  select_chunk(sp, (int)blockIdx.x, smem, dyn);
}

__global__ void __launch_bounds__(SELECT_THREADS) select_kernel(SelectParams sp) {
  __shared__ __attribute__((aligned(16))) char smem[(24 + 16 * 64 + SELECT_FINISH) * 4];
  // dynamic LDS (long rows only): the positions of the final bucket's keys,
  // then the bitmap of a row's selected positions
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  if (sp.done && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(sp.done, sp.done_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  int32_t* cpos = sp.bm_bits > 0 ? reinterpret_cast<int32_t*>(dyn) : nullptr;
  uint32_t* bm = sp.bm_bits > 0 ? reinterpret_cast<uint32_t*>(dyn + SELECT_FINISH * 4) : nullptr;
  const PostItem it = sp.items[blockIdx.x];
  if (sp.n_chunks > 0 && sel_chunked(it.L)) return;  // the chunk launches select it
  const uint32_t* hist = (sp.hist && it.hist_slot >= 0) ? sp.hist + (int64_t)it.hist_slot * HIST_BINS : nullptr;
  select_topk<SELECT_KPT>(sp.pbar + it.pbar_off, it.L, it.K, sp.idx_out + it.idx_off, smem, hist, bm, cpos,
                          sp.bm_bits);
}

// ==========================================================================
// recallable index: sinks + stored important positions + recent tokens
// ==========================================================================
// The per-head index of a draft step keeps the sink tokens, the important
// history positions picked by the last verify's scores, and the recent tokens
// (arxiv.org 2607.27735 as rendered on bittide.aicompass.dev, "全局的稀疏一瞥",
// section 方法, Figure 3 caption).  It is a set over positions [0, L): one
// workgroup per (request, KV head) marks its members in an LDS bitmap -- sinks
// and recent tokens by interval arithmetic, stored entries with LDS atomics, so
// any order and any duplicates in the stored list are fine -- then ranks the
// set bits with one block scan and writes the members ascending, followed by
// -1 up to the output length.
constexpr int RECALL_THREADS = 256;

// Bits of the 32-position word starting at `lo` that fall in [a, b).
__device__ __forceinline__ uint32_t span_bits(int lo, int a, int b) {
  const int x = min(max(a - lo, 0), 32), y = min(max(b - lo, 0), 32);
  if (y <= x) return 0u;
  const uint32_t upto_y = y >= 32 ? 0xffffffffu : ((1u << y) - 1u);
  const uint32_t below_x = x >= 32 ? 0xffffffffu : ((1u << x) - 1u);
  return upto_y & ~below_x;
}

__global__ void __launch_bounds__(RECALL_THREADS) recall_kernel(RecallParams rp) {
  extern __shared__ __attribute__((aligned(16))) uint32_t bitmap[];
  const int r = blockIdx.x / rp.Hkv;
  const int g = blockIdx.x - r * rp.Hkv;
  const RecallReq q = rp.reqs[r];
  const int L = q.L;
  const int nw = (L + 31) >> 5;
  uint32_t* wsum = bitmap + ((nw + 3) & ~3);
  const int s_end = min(rp.n_sink, L);
  const int r_begin = max(s_end, L - min(rp.n_recent, L));
  for (int w = threadIdx.x; w < nw; w += RECALL_THREADS)
    bitmap[w] = span_bits(w * 32, 0, s_end) | span_bits(w * 32, r_begin, L);
  __syncthreads();
  const int32_t* in = rp.idx_in + q.in_off + (int64_t)g * q.in_count;
  for (int t = threadIdx.x; t < q.in_count; t += RECALL_THREADS) {
    const int32_t p = in[t];
    if (p >= 0 && p < L) atomicOr(&bitmap[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // each thread owns a run of consecutive words, so its members are a run of
  // consecutive output entries starting at its exclusive prefix
  const int per = (nw + RECALL_THREADS - 1) / RECALL_THREADS;
  const int w0 = min(nw, (int)threadIdx.x * per), w1 = min(nw, w0 + per);
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(bitmap[w]);
  uint32_t total;
  uint32_t pos = block_exclusive_scan(c, wsum, &total);
  int32_t* out = rp.idx_out + q.out_off + (int64_t)g * q.out_count;
  const uint32_t cap = (uint32_t)q.out_count;
  for (int w = w0; w < w1; ++w) {
    uint32_t b = bitmap[w];
    while (b) {
      const int bit = __ffs(b) - 1;
      if (pos < cap) out[pos] = w * 32 + bit;
      ++pos;
      b &= b - 1u;
    }
  }
  for (uint32_t t = total + threadIdx.x; t < cap; t += RECALL_THREADS) out[t] = -1;
}

// ==========================================================================
// quality of an index list for one query row
// ==========================================================================
// How much of a query row's exact attention an index list captures: the
// softmax mass on the list's positions (attention coverage) and the share of
// the row's exact top-T positions the list holds (recall), the two measures
// by which the review of SparseSpec compares PillarAttn with Quest (核心方法 /
// PillarAttn).  One workgroup per (request, query head h): the list of KV head
// h / G is marked in an LDS bitmap (repeats count once, entries outside [0, L)
// name no position), the row's softmax p = exp(logit - LSE) goes to the
// workspace while the marked positions' mass is summed, and the top-T of p is
// chosen with the same radix selection as PillarAttn's top-K.
constexpr int QUALITY_THREADS = SELECT_THREADS;
constexpr int QUALITY_BATCH = 8;
constexpr size_t SELECT_SMEM = (24 + 16 * 64 + SELECT_FINISH) * 4;

__global__ void __launch_bounds__(QUALITY_THREADS) quality_kernel(QualityParams qp) {
  extern __shared__ __attribute__((aligned(16))) uint32_t member[];
  const int r = blockIdx.x / qp.Hq;
  const int h = blockIdx.x - r * qp.Hq;
  const int g = h / qp.G;
  const QualityReq q = qp.reqs[r];
  const int L = q.L;
  const int nw = (L + 31) >> 5;
  const size_t bitmap_bytes = ((size_t)nw * 4 + 15) / 16 * 16;
  char* sel_smem = reinterpret_cast<char*>(member) + bitmap_bytes;
  float* red = reinterpret_cast<float*>(sel_smem + SELECT_SMEM);  // [QUALITY_THREADS / 64]
  const int tid = threadIdx.x;
  for (int w = tid; w < nw; w += QUALITY_THREADS) member[w] = 0u;
  __syncthreads();
  // loads are issued QUALITY_BATCH at a time, so a row costs one round trip
  // per batch rather than per element
  const int32_t* lst = qp.list + q.list_off + (int64_t)g * q.n;
  for (int t0 = 0; t0 < q.n; t0 += QUALITY_BATCH * QUALITY_THREADS) {
    int32_t pos[QUALITY_BATCH];
#pragma unroll
    for (int u = 0; u < QUALITY_BATCH; ++u) {
      const int t = t0 + u * QUALITY_THREADS + tid;
      pos[u] = t < q.n ? lst[t] : -1;
    }
#pragma unroll
    for (int u = 0; u < QUALITY_BATCH; ++u)
      if (pos[u] >= 0 && pos[u] < L) atomicOr(&member[pos[u] >> 5], 1u << (pos[u] & 31));
  }
  __syncthreads();
  const float* lg = qp.logits + q.logits_off + ((int64_t)qp.row * qp.Hq + h) * L;
  const float lse = qp.lse[(int64_t)q.lse_row * qp.Hq + h];
  float* p = qp.p + q.p_off + (int64_t)h * ((L + 3) & ~3);
  float cov = 0.f;
  for (int j0 = 0; j0 < L; j0 += QUALITY_BATCH * QUALITY_THREADS) {
    float l[QUALITY_BATCH];
#pragma unroll
    for (int u = 0; u < QUALITY_BATCH; ++u) {
      const int j = j0 + u * QUALITY_THREADS + tid;
      l[u] = j < L ? lg[j] : NEG_INF;
    }
#pragma unroll
    for (int u = 0; u < QUALITY_BATCH; ++u) {
      const int j = j0 + u * QUALITY_THREADS + tid;
      if (j < L) {
        const float v = (l[u] == NEG_INF || lse == NEG_INF) ? 0.f : fast_exp2((l[u] - lse) * LOG2E);
        p[j] = v;
        if ((member[j >> 5] >> (j & 31)) & 1u) cov += v;
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) cov += __shfl_xor(cov, off);
  if ((tid & 63) == 0) red[tid >> 6] = cov;
  __syncthreads();  // also orders the p row's stores before the selection reads it
  int32_t* top = qp.top + ((int64_t)r * qp.Hq + h) * qp.T;
  select_topk<SELECT_KPT>(p, L, qp.T, top, sel_smem);
  __syncthreads();
  if (tid < 64) {
    float c = 0.f;
    for (int w = tid; w < QUALITY_THREADS / 64; w += 64) c += red[w];
    int hits = 0;
    for (int t = tid; t < qp.T; t += 64) {
      const int32_t pos = top[t];
      if (pos >= 0 && pos < L) hits += (int)((member[pos >> 5] >> (pos & 31)) & 1u);
    }
    for (int off = 32; off > 0; off >>= 1) {
      c += __shfl_xor(c, off);
      hits += __shfl_xor(hits, off);
    }
    if (tid == 0) {
      qp.coverage[(int64_t)r * qp.Hq + h] = c;
      qp.recall[(int64_t)r * qp.Hq + h] = (float)hits / (float)qp.T;
    }
  }
}

// ==========================================================================
// host-side shapes and launchers
// ==========================================================================
static int group_template(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 5 ? 5 : 8; }

size_t attn_smem_bytes(int dtype, int head_dim, int G, int nthr, bool mfma, bool valu,
                       int max_chunk) {
  size_t s = 16;
  if (mfma)  // stage ring, logits staging, the slots of the longest chunk padded to whole tiles
    s = std::max(s, (head_dim == 128 ? dma_smem_bytes<128>() : dma_smem_bytes<64>()) +
                        logit_stage_bytes(nthr / 64 - 1) +
                        (size_t)(max_chunk + DMA_TT - 1) / DMA_TT * DMA_TT * 4);
  if (valu) {
    const int GM = group_template(G);
    const int E = dtype == 0 ? 8 : 4;
    const int LPR = head_dim / E;
    const int TB = (nthr / LPR) * 4;
    const size_t v = (size_t)DRAFT_MAX_CHUNK * 4 + (size_t)GM * TB * 4 + 3 * GM * 4 +
                     (size_t)(nthr / 64) * GM * head_dim * 4;
    s = std::max(s, v);
  }
  return s;
}

// Workgroups of a persistent launch: as many as are resident at once (the
// occupancy of this kernel, block size and LDS times the CU count), at most
// one per item.  Cached per (device, kernel, block size, LDS bytes).
static int resident_grid(const void* kernel, int nthr, size_t smem, int nitems) {
  struct Entry {
    int dev;
    const void* kernel;
    int nthr;
    size_t smem;
    int blocks;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nitems;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.dev == dev && e.kernel == kernel && e.nthr == nthr && e.smem == smem)
      return std::min(nitems, e.blocks);
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nthr, smem) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      per_cu < 1 || cus < 1) {
    (void)hipGetLastError();
    return nitems;  // one workgroup per item still drains the plan
  }
  cache.push_back(Entry{dev, kernel, nthr, smem, per_cu * cus});
  return std::min(nitems, per_cu * cus);
}

template <int D, typename T>
static hipError_t launch_attn_g(const AttnParams& p, int nitems, int nthr, size_t smem, bool draft,
                                hipStream_t st) {
  const int G = p.G;
#define SPA_ATTN(GMV)                                                                           \
  do {                                                                                          \
    const void* kern = draft ? reinterpret_cast<const void*>(&attn_kernel_draft<D, T, GMV>)     \
                             : reinterpret_cast<const void*>(&attn_kernel<D, T, GMV>);          \
    const int grid = resident_grid(kern, nthr, smem, nitems);                                   \
    if (draft)                                                                                  \
      hipLaunchKernelGGL((attn_kernel_draft<D, T, GMV>), dim3(grid), dim3(nthr), smem, st, p);   \
    else                                                                                        \
      hipLaunchKernelGGL((attn_kernel<D, T, GMV>), dim3(grid), dim3(nthr), smem, st, p);         \
    return hipGetLastError();                                                                   \
  } while (0)
  if constexpr (sizeof(T) == 2) {
    SPA_ATTN(1);  // the MFMA path does not depend on the group template
  } else {
    if (G <= 1) SPA_ATTN(1);
    if (G <= 2) SPA_ATTN(2);
    if (G <= 4) SPA_ATTN(4);
    if (G <= 5) SPA_ATTN(5);
    SPA_ATTN(8);
  }
#undef SPA_ATTN
}

hipError_t launch_attn(const AttnParams& params, int dtype, int head_dim, int nitems, int nthr,
                       size_t smem, bool draft, hipStream_t st) {
  if (nitems == 0) return hipSuccess;
  AttnParams p = params;
  p.n_items = nitems;
  // workgroups start on their own item when two fit per CU (measured; with one
  // workgroup per CU, drawing every item was 1.5% faster)
  p.first_static = nthr <= 256 ? 1 : 0;
  if (dtype == 0) {
    if (head_dim == 128) return launch_attn_g<128, uint16_t>(p, nitems, nthr, smem, draft, st);
    return launch_attn_g<64, uint16_t>(p, nitems, nthr, smem, draft, st);
  }
  if (head_dim == 128) return launch_attn_g<128, float>(p, nitems, nthr, smem, draft, st);
  return launch_attn_g<64, float>(p, nitems, nthr, smem, draft, st);
}

hipError_t launch_select_count(const SelectParams& sp, hipStream_t st) {
  if (sp.n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(select_count_kernel, dim3(sp.n_chunks), dim3(SELECT_THREADS), 0, st, sp);
  return hipGetLastError();
}

hipError_t launch_select_chunks(const SelectParams& sp, hipStream_t st) {
  if (sp.n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(select_chunk_kernel, dim3(sp.n_chunks), dim3(SELECT_THREADS), (size_t)SEL_CAND_CAP * 8,
                     st, sp);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& sp, int nitems, hipStream_t st) {
  if (nitems == 0) return hipSuccess;
  const size_t dyn = sp.bm_bits > 0 ? SELECT_FINISH * 4 + (size_t)sp.bm_bits / 8 : 0;
  hipLaunchKernelGGL(select_kernel, dim3(nitems), dim3(SELECT_THREADS), dyn, st, sp);
  return hipGetLastError();
}

size_t quality_smem_bytes(int max_len) {
  const size_t bitmap = ((size_t)(max_len + 31) / 32 * 4 + 15) / 16 * 16;
  return bitmap + SELECT_SMEM + (QUALITY_THREADS / 64) * 4;
}

hipError_t launch_quality(const QualityParams& qp, int nblocks, size_t smem, hipStream_t st) {
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quality_kernel, dim3(nblocks), dim3(QUALITY_THREADS), smem, st, qp);
  return hipGetLastError();
}

size_t recall_smem_bytes(int max_len) {
  const size_t nw = ((size_t)(max_len + 31) / 32 + 3) / 4 * 4;
  return (nw + RECALL_THREADS / 64) * 4;
}

hipError_t launch_recall(const RecallParams& rp, int nblocks, size_t smem, hipStream_t st) {
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(recall_kernel, dim3(nblocks), dim3(RECALL_THREADS), smem, st, rp);
  return hipGetLastError();
}

// Releases a plan buffer once the launch before it on the stream has ended.
__global__ void __launch_bounds__(64) release_kernel(uint64_t* done, uint64_t val) {
  if (threadIdx.x == 0) __hip_atomic_store(done, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_release(uint64_t* done, uint64_t val, hipStream_t st) {
  hipLaunchKernelGGL(release_kernel, dim3(1), dim3(64), 0, st, done, val);
  return hipGetLastError();
}

size_t post_smem_bytes(int avg_terms, int max_nchunk, bool hist) {
  const size_t avg = hist ? post_hist_offset(avg_terms) + (size_t)HIST_BINS * 4
                          : (size_t)(avg_terms * 4 + 7) / 8 * 8 + (size_t)avg_terms * 8;
  const size_t merge = (size_t)2 * MERGE_ROWS * max_nchunk * 4;
  return std::max<size_t>(16, std::max(avg, merge));
}

hipError_t launch_post(const PostParams& p, int dtype, int head_dim, int nitems, size_t smem,
                       hipStream_t st) {
  if (nitems == 0) return hipSuccess;
#define SPA_POST(DV, TV)                                                                         \
  do {                                                                                           \
    if (p.logits_cached)                                                                         \
      hipLaunchKernelGGL((post_kernel<DV, TV, true>), dim3(nitems), dim3(POST_THREADS), smem, st, p); \
    else                                                                                         \
      hipLaunchKernelGGL((post_kernel<DV, TV, false>), dim3(nitems), dim3(POST_THREADS), smem, st, p); \
  } while (0)
  if (dtype == 0) {
    if (head_dim == 128)
      SPA_POST(128, uint16_t);
    else
      SPA_POST(64, uint16_t);
  } else {
    if (head_dim == 128)
      SPA_POST(128, float);
    else
      SPA_POST(64, float);
  }
#undef SPA_POST
  return hipGetLastError();
}

}  // namespace spa
