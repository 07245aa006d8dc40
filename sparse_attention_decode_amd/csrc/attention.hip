// Sparse attention over the selected pages, GQA geometry, split-K.
//
// Vortex paper note, "System design > 1. vFlow": after selection, exact
// softmax attention runs on the chosen blocks only. The pages' backend reuses
// existing attention kernels ("System design > 3. Execution backend"); this
// one is written for gfx950 instead: decode over a handful of pages per
// (sequence, KV head) is a pure HBM stream (G flop per byte), so it runs on
// the vector ALUs, one wave per work item, with no LDS round trip.
//
// Work item = (sequence b, KV head g, split s); the split streams selected
// pages [s*pps, min(count, (s+1)*pps)). Pages are walked as 16-token chunks.
// A chunk is read with 16-byte loads, lane l covering bytes [16 l, 16 l + 16)
// of every 1 KB of the chunk, so each load instruction is 1 KB contiguous.
// That puts each token row across LPR = Dk / E lanes (E elements per 16 B) and
// TPI = 64 / LPR tokens in one instruction. q.k is a per-lane partial dot
// reduced over the LPR lanes with DPP; each group of LPR lanes ("row") keeps
// its own online-softmax state (m, l, o) for the tokens it holds, so V needs
// no cross-lane traffic. Rows are merged once at the end of the split.
// Logits are kept in log2 units (q pre-scaled by sm_scale * log2 e).
// The next chunk's loads are issued before the current chunk is consumed.
#include "vx_internal.h"

namespace vx {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

template <typename QT, typename KV, int G, int DK, int P>
__global__ __launch_bounds__(256) void attn_gqa_kernel(
    Meta m, int hkv, const QT* __restrict__ q, const KV* __restrict__ kp,
    const KV* __restrict__ vp, const int32_t* __restrict__ sel, int stride,
    const int32_t* __restrict__ sel_count, float qscale, int S, int pps,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using T = KVTraits<KV>;
  constexpr int E = T::E;
  constexpr int LPR = DK / E;      // lanes per token row
  constexpr int TPI = 64 / LPR;    // tokens per load instruction
  constexpr int CT = 16;           // tokens per chunk
  constexpr int CH = CT / TPI;     // load instructions per chunk
  constexpr int CPP = P / CT;      // chunks per page
  constexpr bool kDot2 = sizeof(KV) == 2 && sizeof(QT) == 2;
  static_assert(64 % LPR == 0 && CT % TPI == 0 && P % CT == 0, "layout");

  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int hq = hkv * G;
  if (item >= m.batch * hkv * S) return;
  const int s = item % S;
  const int bg = item / S;
  const int b = bg / hkv, g = bg % hkv;
  const int row = lane / LPR;          // which token of each load this lane holds
  const int dofs = (lane % LPR) * E;   // first dim this lane holds

  const int L = seq_len_clamped(m, b);
  const int cap = m.indptr[b + 1] - m.indptr[b];
  const int count = cap > 0 ? min(sel_count[bg], stride) : 0;
  const int p0 = s * pps;
  const int np = max(0, min(count, p0 + pps) - p0);

  // Page list of this split, one page per lane: physical id and valid tokens.
  int my_phys = 0, my_nv = 0;
  if (lane < np) {
    int lp = sel[(size_t)bg * stride + p0 + lane];
    lp = lp < 0 ? 0 : (lp >= cap ? cap - 1 : lp);
    my_phys = phys_page(m, m.indptr[b] + lp);
    my_nv = max(0, min(P, L - lp * P));
  }

  // Query rows of the group, pre-scaled into log2 units.
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

  const int nchunks = np * CPP;
  const size_t head_stride = (size_t)P * DK;  // elements of one (page, head)

  auto chunk_base = [&](int c, int& nv_chunk) -> size_t {
    const int pi = c / CPP, sub = c % CPP;
    const int phys = __builtin_amdgcn_readlane(my_phys, pi);
    nv_chunk = __builtin_amdgcn_readlane(my_nv, pi) - sub * CT;
    return ((size_t)phys * hkv + g) * head_stride + (size_t)sub * CT * DK;
  };
  auto load_chunk = [&](int c, u32x4* kr, u32x4* vr) {
    int nvc;
    const size_t base = chunk_base(c, nvc);
    if (nvc <= 0) return;
    const u32x4* kc = (const u32x4*)(kp + base);
    const u32x4* vc = (const u32x4*)(vp + base);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      kr[i] = __builtin_nontemporal_load(kc + i * 64 + lane);
      vr[i] = __builtin_nontemporal_load(vc + i * 64 + lane);
    }
  };
  auto consume = [&](int c, const u32x4* kr, const u32x4* vr) {
    int nvc;
    (void)chunk_base(c, nvc);
    if (nvc <= 0) return;
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

  u32x4 kA[CH], vA[CH], kB[CH], vB[CH];
  if (nchunks > 0) load_chunk(0, kA, vA);
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) load_chunk(c + 1, kB, vB);
    consume(c, kA, vA);
    if (c + 1 < nchunks) {
      if (c + 2 < nchunks) load_chunk(c + 2, kA, vA);
      consume(c + 1, kB, vB);
    }
  }

  // Merge the TPI rows (lanes l, l ^ LPR, l ^ 2 LPR, ...) of every head.
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
      const int head = g * G + h;
      if (S == 1) {
        const float inv = lrow[h] > 0.f ? 1.f / lrow[h] : 0.f;
        float* dst = out + ((size_t)b * hq + head) * DK + dofs;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[e] = o[h][e] * inv;
        if (lse && lane == 0)
          lse[(size_t)b * hq + head] =
              lrow[h] > 0.f ? (mrow[h] + log2f(lrow[h])) * kLn2 : -INFINITY;
      } else {
        const size_t ps = ((size_t)b * hq + head) * S + s;
        float* dst = part_o + ps * DK + dofs;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[e] = o[h][e];
        if (lane == 0) {
          part_ml[2 * ps] = mrow[h];
          part_ml[2 * ps + 1] = lrow[h];
        }
      }
    }
  }
}

// out[b][h] = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - max m).
__global__ __launch_bounds__(64) void merge_kernel(int S, int dv, const float* __restrict__ part_o,
                                                   const float* __restrict__ part_ml,
                                                   float* __restrict__ out,
                                                   float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const float* ml = part_ml + (size_t)bh * S * 2;
  float mmax = kNegBig;
  for (int s = 0; s < S; ++s) mmax = fmaxf(mmax, ml[2 * s]);
  float wsum = 0.f;
  for (int s = 0; s < S; ++s) wsum += ml[2 * s + 1] * __builtin_amdgcn_exp2f(ml[2 * s] - mmax);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int d = threadIdx.x; d < dv; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s)
      acc = fmaf(__builtin_amdgcn_exp2f(ml[2 * s] - mmax), part_o[((size_t)bh * S + s) * dv + d], acc);
    out[(size_t)bh * dv + d] = acc * inv;
  }
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
  dim3 block(256), grid((items + 3) / 4);
  const int G = geo.num_q_heads / hkv;
#define VX_ATTN_CASE(GG)                                                                       \
  case GG:                                                                                     \
    hipLaunchKernelGGL((attn_gqa_kernel<QT, KV, GG, DK, P>), grid, block, 0, st, m, hkv,      \
                       (const QT*)q, (const KV*)k_pool, (const KV*)v_pool, sel, stride, cnt,   \
                       qscale, S, pps, out, lse, po, pml);                                     \
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

template <typename QT, typename KV>
hipError_t launch_t(const Meta& m, const vx_geom& geo, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* sel, int stride, const int32_t* cnt,
                    float qscale, int S, int pps, float* out, float* lse, float* po, float* pml,
                    hipStream_t st) {
  const int dk = geo.head_dim_k, P = m.page_size;
  if (dk == 64 && P == 16)
    return launch_g<QT, KV, 64, 16>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, pps,
                                    out, lse, po, pml, st);
  if (dk == 64 && P == 64)
    return launch_g<QT, KV, 64, 64>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, pps,
                                    out, lse, po, pml, st);
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
                                float* part_o, float* part_ml, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  const float qscale = sm_scale * kLog2e;
  if (g.kv_dtype == VX_F32)
    return launch_t<float, float>(m, g, q, k_pool, v_pool, sel, sel_stride, sel_count, qscale,
                                  num_splits, pages_per_split, out, lse, part_o, part_ml, s);
  return launch_t<uint16_t, uint16_t>(m, g, q, k_pool, v_pool, sel, sel_stride, sel_count, qscale,
                                      num_splits, pages_per_split, out, lse, part_o, part_ml, s);
}

hipError_t launch_merge(int batch, int hq, int dv, int num_splits, const float* part_o,
                        const float* part_ml, float* out, float* lse, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(batch * hq), dim3(64), 0, s, num_splits, dv, part_o,
                     part_ml, out, lse);
  return hipGetLastError();
}

}  // namespace vx
