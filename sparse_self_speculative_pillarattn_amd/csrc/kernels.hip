// kernels.hip -- device code of libspa for gfx950 (CDNA4).
//
// attn_kernel   one work item per workgroup: a verify item (request r, KV head g,
//               token chunk) runs the MFMA tile below; a draft item (r, g, chunk of
//               its index list) runs the VALU gather tile.  Both kinds go through
//               the same launch ("Unified batch scheduler + fused attention
//               kernel", SparseSpec review).
// merge_kernel  split-K partials (O, m, l) of one (request, KV head) -> O, LSE.
// avg_kernel    exact scores exp(logit - LSE) averaged over the draft rows and
//               the GQA group (SparseSpec review, PillarAttn, third bullet).
// select_kernel per (verify request, KV head) top-K of the averaged scores by an
//               MSB-first radix select on the fp32 bit patterns, then an ordered
//               compaction so the list comes out ascending (PillarAttn, fourth
//               bullet).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spa_plan.h"
#include "spa_kernels.h"

namespace spa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
#define NEG_INF (-__builtin_inff())

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int64_t clamp_slot(int32_t s, int64_t n) {
  return s < 0 ? 0 : (s >= n ? n - 1 : (int64_t)s);
}

// 16-byte piece -> floats
template <typename T>
struct Piece;
template <>
struct Piece<uint16_t> {  // bf16
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
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* dst, float v) {
  *dst = (uint16_t)f2bf(v);
}
template <>
__device__ __forceinline__ void store_out<float>(float* dst, float v) {
  *dst = v;
}

// LDS chunk swizzle of the K tile: spreads the 16 rows an MFMA operand read
// touches over all banks.
template <int NCH>
__device__ __forceinline__ int kswz(int tau) {
  return ((tau & 3) | (((tau >> 3) & 3) << 2)) & (NCH - 1);
}

// --------------------------------------------------------------------------
// Verify tile on MFMA (bf16).  Rows rho = i*G + hh (query row i, head hh of the
// group) are split into 16-row tiles, one per wave.  Per 64-token tile:
//   S^T = K * Q^T      (16x16x32 MFMA, A = K rows from LDS, B = Q^T in registers)
//   logits stored, online softmax in registers,
//   O^T += V^T * P^T   (A = V^T from the transposed LDS tile, B = P^T, which is
//                       the S^T accumulator layout repacked to bf16 in place).
// Token order inside a tile is permuted so that the S^T accumulator of two
// 16-token MFMA tiles is exactly the P^T operand of one 32-token PV step and
// every lane owns 4 consecutive positions (vector logits stores).
// --------------------------------------------------------------------------
template <int D>
__device__ void verify_tile_mfma(const AttnParams& p, const WorkItem& it, const ReqDesc& rq,
                                 char* smem) {
  constexpr int NCH = D / 8;   // 16-byte chunks per row
  constexpr int KS = D / 32;   // k-steps of S^T = K Q^T
  constexpr int DT = D / 16;   // d tiles of O^T
  constexpr int TT = VERIFY_TILE;
  constexpr int VTS = TT + 8;  // bf16 elements per transposed V row
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = p.G, Hq = p.Hq, Hkv = p.Hkv;
  const int rows_q = p.k + 1;
  const int R = rows_q * G;
  const int g = it.g;
  const int L = rq.L;
  const int jb = it.begin, je = it.end;

  uint4* Ks = reinterpret_cast<uint4*>(smem);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + TT * NCH * 16);
  int32_t* slots = reinterpret_cast<int32_t*>(smem + TT * NCH * 16 + D * VTS * 2);

  const int32_t* ptr = p.page_table + (int64_t)it.r * p.pt_stride;
  for (int j = jb + tid; j < je; j += nthr) slots[j - jb] = (int32_t)clamp_slot(ptr[j], p.num_slots);

  const int n = lane & 15, q4 = lane >> 4;
  const int rho = wave * 16 + n;
  const bool wave_active = wave * 16 < R;
  const bool row_ok = rho < R;
  const int qi = row_ok ? rho / G : 0;
  const int hh = row_ok ? rho % G : 0;
  const int h = g * G + hh;

  bf16x8 qop[KS];
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)(rq.row0 + qi) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok) v = *reinterpret_cast<const uint4*>(qrow + 8 * (4 * s + q4));
      qop[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run = NEG_INF, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int last_vis = L - rows_q + qi;
  float* lrow = p.logits + rq.off + ((int64_t)qi * Hq + h) * L;
  const float sc = p.sm_scale;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(p.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(p.v_pool);

  for (int t0 = jb; t0 < je; t0 += TT) {
    const int nt = min(TT, je - t0);
    __syncthreads();  // slots ready / previous tile consumed
    for (int pc = tid; pc < TT * NCH; pc += nthr) {
      const int tau = pc / NCH, c = pc % NCH;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (tau < nt) {
        const int64_t slot = slots[t0 - jb + tau];
        v = *reinterpret_cast<const uint4*>(kpool + (slot * Hkv + g) * D + 8 * c);
      }
      Ks[tau * NCH + (c ^ kswz<NCH>(tau))] = v;
    }
    for (int u = tid; u < (TT / 4) * NCH; u += nthr) {
      const int tg = u / NCH, c = u % NCH;
      uint32_t w[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 4 * tg + i;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tau < nt) {
          const int64_t slot = slots[t0 - jb + tau];
          v = *reinterpret_cast<const uint4*>(vpool + (slot * Hkv + g) * D + 8 * c);
        }
        w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xffffu;
        const uint32_t a1 = (w[1][e >> 1] >> sh) & 0xffffu;
        const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xffffu;
        const uint32_t a3 = (w[3][e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(Vt + (8 * c + e) * VTS + 4 * tg) =
            make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      }
    }
    __syncthreads();
    if (!wave_active) continue;

    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int tau = 32 * (t >> 1) + 8 * (n >> 2) + 4 * (t & 1) + (n & 3);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + q4;
        const uint4 kv = Ks[tau * NCH + (c ^ kswz<NCH>(tau))];
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qop[s],
                                                          sacc[t], 0, 0, 0);
      }
    }

    float v[4][4];
    float mx = NEG_INF;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 32 * (t >> 1) + 8 * q4 + 4 * (t & 1) + i;
        float x = sacc[t][i] * sc;
        if (tok >= je || tok > last_vis) x = NEG_INF;
        v[t][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    if (row_ok) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tb = t0 + 32 * (t >> 1) + 8 * q4 + 4 * (t & 1);
        float* dst = lrow + tb;
        if (tb + 4 <= je && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[t][0], v[t][1], v[t][2], v[t][3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + i < je) dst[i] = v[t][i];
        }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f, base = 0.f;
    if (m_new != NEG_INF) {
      alpha = fast_exp2((m_run - m_new) * LOG2E);
      base = m_new * LOG2E;
    }
    float psum = 0.f;
    float pf[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = v[t][i];
        const float e = (x == NEG_INF) ? 0.f : fast_exp2(fmaf(x, LOG2E, -base));
        pf[t][i] = e;
        psum += e;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) oacc[dd] *= alpha;
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)pf[2 * kap][i];
        pb[4 + i] = (__bf16)pf[2 * kap + 1][i];
      }
#pragma unroll
      for (int dd = 0; dd < DT; ++dd) {
        const uint4 vv =
            *reinterpret_cast<const uint4*>(Vt + (16 * dd + n) * VTS + 32 * kap + 8 * q4);
        oacc[dd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pb,
                                                           oacc[dd], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!row_ok) return;
  if (rq.nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)(rq.row0 + qi) * Hq + h) * D;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      const uint32_t b0 = f2bf(oacc[dd][0] * inv), b1 = f2bf(oacc[dd][1] * inv);
      const uint32_t b2 = f2bf(oacc[dd][2] * inv), b3 = f2bf(oacc[dd][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dd + 4 * q4) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
    if (q4 == 0)
      p.lse[(int64_t)(rq.row0 + qi) * Hq + h] = l_tot > 0.f ? m_run + logf(l_tot) : NEG_INF;
  } else {
    const int64_t pr = rq.part_row0 + (int64_t)(g * rq.nsplit + it.split) * R + rho;
    float* po = p.part_o + pr * D;
#pragma unroll
    for (int dd = 0; dd < DT; ++dd)
      *reinterpret_cast<float4*>(po + 16 * dd + 4 * q4) =
          make_float4(oacc[dd][0], oacc[dd][1], oacc[dd][2], oacc[dd][3]);
    if (q4 == 0) {
      p.part_ml[2 * pr] = m_run;
      p.part_ml[2 * pr + 1] = l_tot;
    }
  }
}

// --------------------------------------------------------------------------
// VALU gather tile: the GQA group's G query heads of one query row attend to a
// set of positions -- a draft row's index-list entries [begin, end), or (fp32
// verify) the contiguous positions [begin, end) with a causal limit.  Each K/V
// row is read as 16-byte pieces by LPR consecutive lanes, partial dot products
// are reduced with lane shuffles, the softmax statistics of each block go
// through LDS, and P*V accumulates per lane before a final cross-wave sum.
// --------------------------------------------------------------------------
template <int D, typename T, int GM>
__device__ void gather_tile_valu(const AttnParams& p, const WorkItem& it, const ReqDesc& rq,
                                 char* smem, bool is_list, int qi, int last_vis, float* lrow,
                                 int rho0, int Rr) {
  constexpr int E = Piece<T>::E;   // elements per 16-byte piece
  constexpr int LPR = D / E;       // lanes per K/V row
  constexpr int TPT = 4;           // rows per thread per block
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
  const int G = p.G, Hq = p.Hq, Hkv = p.Hkv, g = it.g;
  const int c = tid % LPR, tl = tid / LPR, NTL = nthr / LPR;
  const int TB = NTL * TPT;
  const int nent = it.end - it.begin;
  const int L = rq.L;

  int32_t* slots = reinterpret_cast<int32_t*>(smem);
  float* scs = reinterpret_cast<float*>(slots + DRAFT_MAX_CHUNK);  // [GM][TB]
  float* st = scs + GM * TB;                                         // m[GM], l[GM], alpha[GM]
  float* red = st + 3 * GM;                                          // [nwaves][GM][D]

  const int32_t* ptr = p.page_table + (int64_t)it.r * p.pt_stride;
  const int32_t* list = is_list ? p.idx + rq.off + (int64_t)g * rq.list_len : nullptr;
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
  const T* qbase = reinterpret_cast<const T*>(p.q) + ((int64_t)(rq.row0 + qi) * Hq + g * G) * D;
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

  for (int b0 = 0; b0 < nent; b0 += TB) {
    int32_t sl[TPT];
    uint4 kr[TPT], vr[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = b0 + tl + NTL * i;
      sl[i] = (t < nent) ? slots[t] : -1;
      kr[i] = make_uint4(0u, 0u, 0u, 0u);
      vr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (sl[i] >= 0) {
        const int64_t off = ((int64_t)sl[i] * Hkv + g) * D + c * E;
        kr[i] = *reinterpret_cast<const uint4*>(kpool + off);
        vr[i] = *reinterpret_cast<const uint4*>(vpool + off);
      }
    }
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
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) a += __shfl_xor(a, off);
        dot[hh] = a;
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
    __syncthreads();
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
    if (rq.nsplit == 1) {
      const int64_t orow = (int64_t)(rq.row0 + qi) * Hq + h;
      store_out<T>(reinterpret_cast<T*>(p.o) + orow * D + d, l > 0.f ? acc / l : 0.f);
      if (d == 0) p.lse[orow] = l > 0.f ? m + logf(l) : NEG_INF;
    } else {
      const int64_t pr = rq.part_row0 + (int64_t)(g * rq.nsplit + it.split) * Rr + rho0 + hh;
      p.part_o[pr * D + d] = acc;
      if (d == 0) {
        p.part_ml[2 * pr] = m;
        p.part_ml[2 * pr + 1] = l;
      }
    }
  }
}

template <int D, typename T, int GM>
__global__ void __launch_bounds__(512) attn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const WorkItem it = p.items[blockIdx.x];
  const ReqDesc rq = p.reqs[it.r];
  if (rq.kind == KIND_VERIFY) {
    if constexpr (sizeof(T) == 2) {
      verify_tile_mfma<D>(p, it, rq, smem);
    } else {
      const int qi = it.qi;
      const int last_vis = rq.L - (p.k + 1) + qi;
      float* lrow = p.logits + rq.off + ((int64_t)qi * p.Hq + it.g * p.G) * rq.L;
      gather_tile_valu<D, T, GM>(p, it, rq, smem, false, qi, last_vis, lrow, qi * p.G,
                                 (p.k + 1) * p.G);
    }
  } else {
    gather_tile_valu<D, T, GM>(p, it, rq, smem, true, 0, 0x7fffffff, nullptr, 0, p.G);
  }
}

// --------------------------------------------------------------------------
// split-K merge: m* = max_s m_s, l* = sum_s l_s e^{m_s - m*},
// O = sum_s e^{m_s - m*} O_s / l*, LSE = m* + ln l*.
// --------------------------------------------------------------------------
template <int D, typename T>
__global__ void __launch_bounds__(256) merge_kernel(MergeParams mp) {
  const MergeItem mi = mp.items[blockIdx.x];
  const ReqDesc rq = mp.reqs[mi.r];
  const int G = mp.G;
  const int rows_q = rq.kind == KIND_VERIFY ? mp.k + 1 : 1;
  const int R = rows_q * G;
  const int ns = rq.nsplit;
  const int64_t base = rq.part_row0 + (int64_t)mi.g * ns * R;
  for (int x = threadIdx.x; x < R * D; x += blockDim.x) {
    const int rho = x / D, d = x % D;
    float mstar = NEG_INF;
    for (int s = 0; s < ns; ++s) mstar = fmaxf(mstar, mp.part_ml[2 * (base + (int64_t)s * R + rho)]);
    float lsum = 0.f, acc = 0.f;
    if (mstar != NEG_INF) {
      for (int s = 0; s < ns; ++s) {
        const int64_t pr = base + (int64_t)s * R + rho;
        const float m = mp.part_ml[2 * pr], l = mp.part_ml[2 * pr + 1];
        const float w = (m == NEG_INF) ? 0.f : fast_exp2((m - mstar) * LOG2E);
        lsum = fmaf(w, l, lsum);
        acc = fmaf(w, mp.part_o[pr * D + d], acc);
      }
    }
    const int qi = rho / G, hh = rho % G;
    const int64_t orow = (int64_t)(rq.row0 + qi) * mp.Hq + mi.g * G + hh;
    store_out<T>(reinterpret_cast<T*>(mp.o) + orow * D + d, lsum > 0.f ? acc / lsum : 0.f);
    if (d == 0) mp.lse[orow] = lsum > 0.f ? mstar + logf(lsum) : NEG_INF;
  }
}

// --------------------------------------------------------------------------
// averaged exact scores: pbar[j] = 1/(n G) sum_i sum_hh exp(logit - LSE)
// --------------------------------------------------------------------------
__global__ void __launch_bounds__(256) avg_kernel(AvgParams ap) {
  __shared__ float lse_s[MAX_AVG_TERMS];
  const AvgItem ai = ap.avg[blockIdx.x];
  const TopkItem ti = ap.topk[ai.t];
  const int G = ap.G, Hq = ap.Hq, n = ap.row_count, a = ap.row_begin;
  const int terms = n * G;
  const int L = ti.L;
  for (int x = threadIdx.x; x < terms; x += blockDim.x) {
    const int i = a + x / G, hh = x % G;
    lse_s[x] = ap.lse[(int64_t)(ti.lse_row0 + i) * Hq + ti.g * G + hh];
  }
  __syncthreads();
  const float inv = 1.f / (float)terms;
  const float* lg = ap.logits + ti.logits_off;
  const int jend = min(ai.j0 + AVG_SPAN, L);
  for (int j = ai.j0 + threadIdx.x; j < jend; j += blockDim.x) {
    float s = 0.f;
    for (int x = 0; x < terms; ++x) {
      const int i = a + x / G, hh = x % G;
      const float l = lg[((int64_t)i * Hq + ti.g * G + hh) * L + j];
      s += (l == NEG_INF) ? 0.f : expf(l - lse_s[x]);
    }
    ap.pbar[ti.pbar_off + j] = s * inv;
  }
}

// --------------------------------------------------------------------------
// top-K by MSB-first radix select over the fp32 bit patterns (scores are >= 0,
// so the unsigned order of the bits is the numeric order), then an ordered
// compaction: every position above the threshold, plus the lowest positions
// equal to it, written ascending.
// --------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) select_kernel(SelectParams sp) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_rem;
  __shared__ uint32_t cnt_eq[16], cnt_take[16];
  __shared__ uint32_t s_base_eq, s_base_take;
  const TopkItem ti = sp.topk[blockIdx.x];
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(sp.pbar + ti.pbar_off);
  const int L = ti.L, K = ti.K;
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = nthr >> 6;
  if (tid == 0) {
    s_prefix = 0u;
    s_rem = (uint32_t)K;
    s_base_eq = 0u;
    s_base_take = 0u;
  }
  uint32_t mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += nthr) hist[b] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int j = tid; j < L; j += nthr) {
      const uint32_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cnt[4], sum = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cnt[i] = hist[255 - 4 * lane - i];
        sum += cnt[i];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const uint32_t excl = incl - sum;
      const uint32_t rem = s_rem;
      if (excl < rem && incl >= rem) {
        uint32_t acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (acc + cnt[i] >= rem) {
            s_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
            s_rem = rem - acc;
            break;
          }
          acc += cnt[i];
        }
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t tau = s_prefix, rem = s_rem;
  int32_t* out = sp.idx + ti.idx_off;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < L; c0 += nthr) {
    const int j = c0 + tid;
    const uint32_t key = j < L ? keys[j] : 0u;
    const bool gt = j < L && key > tau;
    const bool eq = j < L && key == tau;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) cnt_eq[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_rank = s_base_eq + (uint32_t)__popcll(beq & lt_mask);
    for (int w = 0; w < wave; ++w) eq_rank += cnt_eq[w];
    const bool take = gt || (eq && eq_rank < rem);
    const uint64_t btk = __ballot(take);
    if (lane == 0) cnt_take[wave] = (uint32_t)__popcll(btk);
    __syncthreads();
    uint32_t pos = s_base_take + (uint32_t)__popcll(btk & lt_mask);
    for (int w = 0; w < wave; ++w) pos += cnt_take[w];
    if (take && pos < (uint32_t)K) out[pos] = j;
    __syncthreads();
    if (tid == 0) {
      uint32_t te = 0u, tt = 0u;
      for (int w = 0; w < nwaves; ++w) {
        te += cnt_eq[w];
        tt += cnt_take[w];
      }
      s_base_eq += te;
      s_base_take += tt;
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
template <int D, typename T>
static hipError_t launch_attn_g(const AttnParams& p, int nitems, int nthr, size_t smem,
                                hipStream_t st) {
  const int G = p.G;
#define SPA_ATTN(GMV)                                                                       \
  do {                                                                                      \
    hipLaunchKernelGGL((attn_kernel<D, T, GMV>), dim3(nitems), dim3(nthr), smem, st, p);    \
    return hipGetLastError();                                                               \
  } while (0)
  if (G <= 1) SPA_ATTN(1);
  if (G <= 2) SPA_ATTN(2);
  if (G <= 4) SPA_ATTN(4);
  if (G <= 5) SPA_ATTN(5);
  SPA_ATTN(8);
#undef SPA_ATTN
}

hipError_t launch_attn(const AttnParams& p, int dtype, int head_dim, int nitems, int nthr,
                       size_t smem, hipStream_t st) {
  if (nitems == 0) return hipSuccess;
  if (dtype == 0) {
    if (head_dim == 128) return launch_attn_g<128, uint16_t>(p, nitems, nthr, smem, st);
    return launch_attn_g<64, uint16_t>(p, nitems, nthr, smem, st);
  }
  if (head_dim == 128) return launch_attn_g<128, float>(p, nitems, nthr, smem, st);
  return launch_attn_g<64, float>(p, nitems, nthr, smem, st);
}

hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, int nitems,
                        hipStream_t st) {
  if (nitems == 0) return hipSuccess;
  if (dtype == 0) {
    if (head_dim == 128)
      hipLaunchKernelGGL((merge_kernel<128, uint16_t>), dim3(nitems), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((merge_kernel<64, uint16_t>), dim3(nitems), dim3(256), 0, st, p);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((merge_kernel<128, float>), dim3(nitems), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((merge_kernel<64, float>), dim3(nitems), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_avg(const AvgParams& ap, int navg, hipStream_t st) {
  if (navg == 0) return hipSuccess;
  hipLaunchKernelGGL(avg_kernel, dim3(navg), dim3(256), 0, st, ap);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& sp, int ntopk, hipStream_t st) {
  if (ntopk == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3(ntopk), dim3(1024), 0, st, sp);
  return hipGetLastError();
}

}  // namespace spa
