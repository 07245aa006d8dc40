// Sparse attention over the selected pages, GQA geometry, split-K.
//
// Vortex paper note, "System design > 1. vFlow": after selection, exact
// softmax attention runs on the chosen blocks only. The pages' backend reuses
// existing attention kernels ("System design > 3. Execution backend"); this
// one is written for gfx950 instead: decode over a handful of pages per
// (sequence, KV head) is a pure HBM stream (G flop per byte), so it runs on
// the vector ALUs with no LDS round trip for K/V.
//
// One block of 8 waves per (sequence b, KV head g, split s); the split holds
// a balanced share of the selection (all of it when the batch fills the
// GPU). Pages are walked as 16-token chunks, dealt round-robin to the waves;
// each wave loads a batch of chunks, then consumes it. A chunk is read
// with 16-byte loads, lane l covering bytes [16 l, 16 l + 16) of every 1 KB,
// so each load instruction is 1 KB contiguous. That puts each token row
// across LPR = Dk / E lanes (E elements per 16 B) and TPI = 64 / LPR tokens
// in one instruction. q.k is a per-lane partial (v_dot2_f32_bf16 for bf16)
// reduced over the LPR lanes with DPP; each group of LPR lanes ("row") keeps
// its own online-softmax state (m, l, o) for the tokens it holds, so V needs
// no cross-lane traffic. Rows merge inside the wave, waves merge in LDS, and
// splits (if any) merge in merge_kernel. Logits are in log2 units.
#include "attn_mfma.h"

namespace vx {
namespace {


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename KV> struct KVTraits;
template <> struct KVTraits<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void to_f32(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};
template <> struct KVTraits<uint16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void to_f32(const u32x4& w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
};

// Page range of split s among S: balanced over the selection actually used.
__device__ __forceinline__ void split_range(int count, int S, int s, int& p0, int& np) {
  p0 = (int)(((long)count * s) / S);
  np = (int)(((long)count * (s + 1)) / S) - p0;
}

#ifndef VX_ATTN_WAVES
#define VX_ATTN_WAVES 8
#endif
constexpr int kWaves = VX_ATTN_WAVES;  // waves per attention block
#ifndef VX_ATTN_BATCH
#define VX_ATTN_BATCH 1
#endif
constexpr int kBatch = VX_ATTN_BATCH;  // chunks in flight per wave (vector kernel, short rows)

template <typename QT, typename KV, int G, int DK, int P>
__global__ __launch_bounds__(64 * kWaves) void attn_gqa_kernel(
    Meta m, int hkv, const QT* __restrict__ q, const KV* __restrict__ kp,
    const KV* __restrict__ vp, const int32_t* __restrict__ sel, int stride,
    const int32_t* __restrict__ sel_count, float qscale, int S,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using T = KVTraits<KV>;
  constexpr int E = T::E;
  constexpr int LPR = DK / E;      // lanes per token row
  constexpr int TPI = 64 / LPR;    // tokens per load instruction
  constexpr int CT = 16;           // tokens per chunk
  constexpr int CH = CT / TPI;     // load instructions per chunk (per K and per V)
  constexpr int CPP = P / CT;      // chunks per page
  constexpr bool kDot2 = sizeof(KV) == 2 && sizeof(QT) == 2;
  static_assert(64 % LPR == 0 && CT % TPI == 0 && P % CT == 0, "layout");

  static_assert(kMaxPagesPerSplit <= 64 * kWaves, "one page-list entry per thread");
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];
  __shared__ float red_o[kWaves][G][DK];
  __shared__ float red_ml[kWaves][G][2];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hq = hkv * G;
  const int item = blockIdx.x;
  const int s = item % S, bg = item / S;
  const int b = bg / hkv, g = bg % hkv;
  const int row = lane / LPR;
  const int dofs = (lane % LPR) * E;

  const int L = seq_len_clamped(m, b);
  const int cap = m.indptr[b + 1] - m.indptr[b];
  const int count = cap > 0 ? min(sel_count[bg], stride) : 0;
  int p0, np;
  split_range(count, S, s, p0, np);
  np = min(np, kMaxPagesPerSplit);
  if (threadIdx.x < np) {
    int lp = sel[(size_t)bg * stride + p0 + threadIdx.x];
    lp = lp < 0 ? 0 : (lp >= cap ? cap - 1 : lp);
    pg_phys[threadIdx.x] = phys_page(m, m.indptr[b] + lp);
    pg_nv[threadIdx.x] = max(0, min(P, L - lp * P));
  }

  // Query rows of the group (log2 units): packed bf16 pairs for v_dot2, or fp32.
  float qf[G][E];
  uint32_t qp[G][E / 2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const QT* qh = q + ((size_t)b * hq + g * G + h) * DK + dofs;
    if constexpr (kDot2) {
#pragma unroll
      for (int e = 0; e < E / 2; ++e) qp[h][e] = ((const uint32_t*)qh)[e];
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (sizeof(QT) == 2) qf[h][e] = bf16_to_f32(qh[e]) * qscale;
        else qf[h][e] = (float)qh[e] * qscale;
      }
    }
  }

  float mrow[G], lrow[G], o[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mrow[h] = kNegBig;
    lrow[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = 0.f;
  }
  __syncthreads();  // page list ready

  const int nchunks = np * CPP;
  const size_t head_stride = (size_t)P * DK;
  auto chunk_nv = [&](int c) { return pg_nv[c / CPP] - (c % CPP) * CT; };
  auto load_chunk = [&](int c, u32x4* kr, u32x4* vr) {
    const size_t base = ((size_t)pg_phys[c / CPP] * hkv + g) * head_stride + (size_t)(c % CPP) * CT * DK;
    const u32x4* kc = (const u32x4*)(kp + base);
    const u32x4* vc = (const u32x4*)(vp + base);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      kr[i] = __builtin_nontemporal_load(kc + i * 64 + lane);
      vr[i] = __builtin_nontemporal_load(vc + i * 64 + lane);
    }
  };
  // No early exit: an empty chunk is consumed fully masked, so every slot's
  // loads are waited on in one place and the prefetch ring stays pipelined.
  auto consume = [&](int c, const u32x4* kr, const u32x4* vr) {
    const int nvc = chunk_nv(c);
    const bool full = nvc >= CT;
    float z[CH][G];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool valid = full || (i * TPI + row) < nvc;
      if constexpr (kDot2) {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[h][e]),
                                                  __builtin_bit_cast(bf16x2_t, kw[e]), acc, false);
          acc = group_sum<LPR>(acc) * qscale;
          z[i][h] = valid ? acc : -INFINITY;
        }
      } else {
        float kf[E];
        T::to_f32(kr[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(qf[h][e], kf[e], acc);
          acc = group_sum<LPR>(acc);
          z[i][h] = valid ? acc : -INFINITY;
        }
      }
    }
    float pr[CH][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = z[0][h];
#pragma unroll
      for (int i = 1; i < CH; ++i) mx = fmaxf(mx, z[i][h]);
      const float mnew = fmaxf(mrow[h], mx);
      const float alpha = __builtin_amdgcn_exp2f(mrow[h] - mnew);
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        pr[i][h] = __builtin_amdgcn_exp2f(z[i][h] - mnew);
        lsum += pr[i][h];
      }
      lrow[h] = fmaf(lrow[h], alpha, lsum);
      mrow[h] = mnew;
#pragma unroll
      for (int e = 0; e < E; ++e) o[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      float vf[E];
      T::to_f32(vr[i], vf);
      if (!full && (i * TPI + row) >= nvc) {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = fmaf(pr[i][h], vf[e], o[h][e]);
    }
  };

  // Batches of NB chunks (see attn_gqa_mfma_kernel): loads first, then use.
  constexpr int NB = CH >= 8 ? 1 : kBatch;
  const int my_n = nchunks > w ? (nchunks - w + kWaves - 1) / kWaves : 0;
  for (int j0 = 0; j0 < my_n; j0 += NB) {
    u32x4 kr[NB][CH], vr[NB][CH];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      load_chunk(w + min(j0 + u, my_n - 1) * kWaves, kr[u], vr[u]);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (j0 + u < my_n) consume(w + (j0 + u) * kWaves, kr[u], vr[u]);
  }

  // Merge the TPI rows of each head inside the wave (lanes l ^ LPR, ...).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) {
      const float mo = __shfl_xor(mrow[h], x);
      const float lo = __shfl_xor(lrow[h], x);
      const float mnew = fmaxf(mrow[h], mo);
      const float a = __builtin_amdgcn_exp2f(mrow[h] - mnew);
      const float bsc = __builtin_amdgcn_exp2f(mo - mnew);
      lrow[h] = lrow[h] * a + lo * bsc;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float oo = __shfl_xor(o[h][e], x);
        o[h][e] = o[h][e] * a + oo * bsc;
      }
      mrow[h] = mnew;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) red_o[w][h][dofs + e] = o[h][e];
      if (lane == 0) {
        red_ml[w][h][0] = mrow[h];
        red_ml[w][h][1] = lrow[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves: thread -> (head, 4 dims).
  for (int t = threadIdx.x; t < G * DK / 4; t += blockDim.x) {
    const int h = t / (DK / 4), d = (t % (DK / 4)) * 4;
    float mmax = kNegBig;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) mmax = fmaxf(mmax, red_ml[v][h][0]);
    float lsum = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float wt = __builtin_amdgcn_exp2f(red_ml[v][h][0] - mmax);
      lsum = fmaf(red_ml[v][h][1], wt, lsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(red_o[v][h][d + e], wt, acc[e]);
    }
    const int head = g * G + h;
    if (S == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float4* dst = (float4*)(out + ((size_t)b * hq + head) * DK + d);
      *dst = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      if (lse && d == 0)
        lse[(size_t)b * hq + head] = lsum > 0.f ? (mmax + log2f(lsum)) * kLn2 : -INFINITY;
    } else {
      const size_t ps = ((size_t)b * hq + head) * S + s;
      *(float4*)(part_o + ps * DK + d) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      if (d == 0) {
        part_ml[2 * ps] = mmax;
        part_ml[2 * ps + 1] = lsum;
      }
    }
  }
}

// The bf16, Dk = Dv = 128 path on the matrix cores: mfma_attend in attn_mfma.h.
template <int G, int P, int NW>
__global__ __launch_bounds__(64 * NW) void attn_gqa_mfma_kernel(
    Meta m, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const int32_t* __restrict__ sel, int stride,
    const int32_t* __restrict__ sel_count, float qscale, int S, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  static_assert(kMaxPagesPerSplit <= 64 * NW, "one page-list entry per thread");
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];
  __shared__ MfmaShared<G, NW> sm;

  const int item = blockIdx.x;
  const int s = item % S, bg = item / S;
  const int b = bg / hkv, g = bg % hkv;
  const int L = seq_len_clamped(m, b);
  const int cap = m.indptr[b + 1] - m.indptr[b];
  const int count = cap > 0 ? min(sel_count[bg], stride) : 0;
  int p0, np;
  split_range(count, S, s, p0, np);
  np = min(np, kMaxPagesPerSplit);
  if (threadIdx.x < np) {
    int lp = sel[(size_t)bg * stride + p0 + threadIdx.x];
    lp = lp < 0 ? 0 : (lp >= cap ? cap - 1 : lp);
    pg_phys[threadIdx.x] = phys_page(m, m.indptr[b] + lp);
    pg_nv[threadIdx.x] = max(0, min(P, L - lp * P));
  }
  u32x4 qa[4];
  mfma_load_q<G>(q, b, g, hkv, qa);
  __syncthreads();  // page list ready
  mfma_attend<G, P, NW>(sm, pg_phys, pg_nv, np, b, g, hkv, qa, kp, vp, qscale, S, s, out, lse,
                            part_o, part_ml);
}

// out[b][h] = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - max m).
// One block per (sequence, head), one thread per 4 value columns.
__global__ __launch_bounds__(128) void merge_kernel(int S, int dv, const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const float* ml = part_ml + (size_t)bh * S * 2;
  float mmax = kNegBig;
  for (int s = 0; s < S; ++s) mmax = fmaxf(mmax, ml[2 * s]);
  const int d = 4 * threadIdx.x;
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* po = part_o + (size_t)bh * S * dv + d;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float wt = __builtin_amdgcn_exp2f(ml[2 * s] - mmax);
    wsum = fmaf(ml[2 * s + 1], wt, wsum);
    if (d < dv) {
      const float4 x = *(const float4*)(po + (size_t)s * dv);
      acc.x = fmaf(x.x, wt, acc.x); acc.y = fmaf(x.y, wt, acc.y);
      acc.z = fmaf(x.z, wt, acc.z); acc.w = fmaf(x.w, wt, acc.w);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (d < dv)
    *(float4*)(out + (size_t)bh * dv + d) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse && threadIdx.x == 0)
    lse[bh] = wsum > 0.f ? (mmax + log2f(wsum)) * kLn2 : -INFINITY;
}

template <typename QT, typename KV, int DK, int P>
hipError_t launch_g(const Meta& m, const vx_geom& geo, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* sel, int stride, const int32_t* cnt,
                    float qscale, int S, int pps, float* out, float* lse, float* po, float* pml,
                    hipStream_t st) {
  const int hkv = geo.num_kv_heads;
  const int items = m.batch * hkv * S;
  dim3 block(64 * kWaves), grid(items);
  const int G = geo.num_q_heads / hkv;
#define VX_ATTN_CASE(GG)                                                                       \
  case GG:                                                                                     \
    hipLaunchKernelGGL((attn_gqa_kernel<QT, KV, GG, DK, P>), grid, block, 0, st, m, hkv,      \
                       (const QT*)q, (const KV*)k_pool, (const KV*)v_pool, sel, stride, cnt,   \
                       qscale, S, out, lse, po, pml);                                          \
    break;
  switch (G) {
    VX_ATTN_CASE(1)
    VX_ATTN_CASE(2)
    VX_ATTN_CASE(4)
    VX_ATTN_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef VX_ATTN_CASE
  return hipGetLastError();
}

template <int G, int P>
hipError_t launch_mfma_g(const Meta& m, int hkv, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* sel, int stride, const int32_t* cnt,
                         float qscale, int S, float* out, float* lse, float* po, float* pml,
                         int max_pages, hipStream_t st) {
  dim3 grid(m.batch * hkv * S);
  if constexpr (G <= 4) {
    if (gqa_attn_waves(G, max_pages) == 16) {
      hipLaunchKernelGGL((attn_gqa_mfma_kernel<G, P, 16>), grid, dim3(1024), 0, st, m, hkv,
                         (const uint16_t*)q, (const uint16_t*)k_pool, (const uint16_t*)v_pool, sel,
                         stride, cnt, qscale, S, out, lse, po, pml);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_gqa_mfma_kernel<G, P, 8>), grid, dim3(512), 0, st, m, hkv,
                     (const uint16_t*)q, (const uint16_t*)k_pool, (const uint16_t*)v_pool, sel,
                     stride, cnt, qscale, S, out, lse, po, pml);
  return hipGetLastError();
}

template <int P>
hipError_t launch_mfma(const Meta& m, const vx_geom& geo, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* sel, int stride, const int32_t* cnt,
                       float qscale, int S, float* out, float* lse, float* po, float* pml,
                       int max_pages, hipStream_t st) {
  const int hkv = geo.num_kv_heads;
  switch (geo.num_q_heads / hkv) {
    case 1: return launch_mfma_g<1, P>(m, hkv, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out,
                                       lse, po, pml, max_pages, st);
    case 2: return launch_mfma_g<2, P>(m, hkv, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out,
                                       lse, po, pml, max_pages, st);
    case 4: return launch_mfma_g<4, P>(m, hkv, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out,
                                       lse, po, pml, max_pages, st);
    case 8: return launch_mfma_g<8, P>(m, hkv, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out,
                                       lse, po, pml, max_pages, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename QT, typename KV>
hipError_t launch_t(const Meta& m, const vx_geom& geo, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* sel, int stride, const int32_t* cnt,
                    float qscale, int S, int pps, float* out, float* lse, float* po, float* pml,
                    int max_pages, hipStream_t st) {
  const int dk = geo.head_dim_k, P = m.page_size;
  if (dk == 64 && P == 16)
    return launch_g<QT, KV, 64, 16>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, pps,
                                    out, lse, po, pml, st);
  if (dk == 64 && P == 64)
    return launch_g<QT, KV, 64, 64>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, pps,
                                    out, lse, po, pml, st);
#ifndef VX_GQA_FORCE_VALU
  if constexpr (sizeof(KV) == 2) {
    if (dk == 128 && P == 16)
      return launch_mfma<16>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out, lse,
                             po, pml, max_pages, st);
    if (dk == 128 && P == 64)
      return launch_mfma<64>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out, lse,
                             po, pml, max_pages, st);
  }
#endif
  if (dk == 128 && P == 16)
    return launch_g<QT, KV, 128, 16>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, pps,
                                     out, lse, po, pml, st);
  if (dk == 128 && P == 64)
    return launch_g<QT, KV, 128, 64>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, pps,
                                     out, lse, po, pml, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention_gqa(const Meta& m, const vx_geom& g, const void* q,
                                const void* k_pool, const void* v_pool, const int32_t* sel,
                                int sel_stride, const int32_t* sel_count, float sm_scale,
                                int num_splits, int pages_per_split, float* out, float* lse,
                                float* part_o, float* part_ml, int max_pages, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  const float qscale = sm_scale * kLog2e;
  if (g.kv_dtype == VX_F32)
    return launch_t<float, float>(m, g, q, k_pool, v_pool, sel, sel_stride, sel_count, qscale,
                                  num_splits, pages_per_split, out, lse, part_o, part_ml, max_pages,
                                  s);
  return launch_t<uint16_t, uint16_t>(m, g, q, k_pool, v_pool, sel, sel_stride, sel_count, qscale,
                                      num_splits, pages_per_split, out, lse, part_o, part_ml,
                                      max_pages, s);
}

hipError_t launch_merge(int batch, int hq, int dv, int num_splits, const float* part_o,
                        const float* part_ml, float* out, float* lse, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(batch * hq), dim3((dv / 4 + 63) / 64 * 64), 0, s,
                     num_splits, dv, part_o, part_ml, out, lse);
  return hipGetLastError();
}

}  // namespace vx
