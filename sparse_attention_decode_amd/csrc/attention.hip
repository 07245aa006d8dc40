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
// GPU); splits (if any) merge in merge_kernel. The vector body (fp32 keys or
// Dk = 64) is vec_attend in attn_vec.h, the bf16 Dk = 128 body mfma_attend
// in attn_mfma.h; the whole-step kernels call the same bodies.
#include "attn_mfma.h"
#include "attn_vec.h"

namespace vx {
namespace {


// Page range of split s among S: balanced over the selection actually used.
__device__ __forceinline__ void split_range(int count, int S, int s, int& p0, int& np) {
  p0 = (int)(((long)count * s) / S);
  np = (int)(((long)count * (s + 1)) / S) - p0;
}

template <typename QT, typename KV, int G, int DK, int P>
__global__ __launch_bounds__(64 * kVecWaves) void attn_gqa_kernel(
    Meta m, int hkv, const QT* __restrict__ q, const KV* __restrict__ kp,
    const KV* __restrict__ vp, const int32_t* __restrict__ sel, int stride,
    const int32_t* __restrict__ sel_count, float qscale, int S,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  static_assert(kMaxPagesPerSplit <= 64 * kVecWaves, "one page-list entry per thread");
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];
  __shared__ VecShared<G, DK> sm;

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
  VecQuery<QT, KV, G> vq;
  vec_load_q<QT, KV, G, DK>(q, b, g, hkv, qscale, vq);
  __syncthreads();  // page list ready
  vec_attend<QT, KV, G, DK, P>(sm, pg_phys, pg_nv, np, b, g, hkv, vq, kp, vp, qscale, S, s, out,
                               lse, part_o, part_ml);
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

// out[b][h] = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - max m)
// (merge_row). One block per (sequence, head), one thread per 4 value
// columns.
__global__ __launch_bounds__(128) void merge_kernel(int S, int dv, const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int d = 4 * threadIdx.x;
  if (d >= dv) return;
  merge_row(S, dv, part_o + (size_t)bh * S * dv + d, part_ml + (size_t)bh * S * 2,
            out + (size_t)bh * dv + d, (lse && threadIdx.x == 0) ? lse + bh : nullptr);
}

template <typename QT, typename KV, int DK, int P>
hipError_t launch_g(const Meta& m, const vx_geom& geo, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* sel, int stride, const int32_t* cnt,
                    float qscale, int S, int pps, float* out, float* lse, float* po, float* pml,
                    hipStream_t st) {
  const int hkv = geo.num_kv_heads;
  const int items = m.batch * hkv * S;
  dim3 block(64 * kVecWaves), grid(items);
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
  if constexpr (sizeof(KV) == 2) {
    if (dk == 128 && P == 16)
      return launch_mfma<16>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out, lse,
                             po, pml, max_pages, st);
    if (dk == 128 && P == 64)
      return launch_mfma<64>(m, geo, q, k_pool, v_pool, sel, stride, cnt, qscale, S, out, lse,
                             po, pml, max_pages, st);
  }
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
