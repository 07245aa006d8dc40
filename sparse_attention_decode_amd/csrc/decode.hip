// The whole decode step for one (sequence, KV head) segment in one block:
// indexer (newest-page refresh, scores, top-k) then exact attention over the
// chosen pages. GQA, bf16, Dk = Dv = 128, one split per segment.
//
// Vortex paper note, "System design > 1. vFlow": cache stage, indexer and
// sparse attention form the step; "System design > 3. Execution backend":
// sequence-local operators are fused greedily. The selection of a segment
// feeds only that segment's attention, so a block that has just selected
// can attend at once: the chosen ids and the physical page of every entry
// are already in its LDS (no kernel boundary, no reload of the selection or
// of the page table). BOUNDS: the Quest-style indexer (page key bounds) in
// place of the centroids. bf16 keys with Dk = 128 attend on the matrix cores
// (mfma_attend); fp32 keys or Dk = 64 on the vector ALUs (vec_attend), the
// bodies of the stand-alone attention kernels, so the bits are the same.
#include "attn_mfma.h"
#include "attn_vec.h"
#include "index_seg.h"

namespace vx {
namespace {

template <int G, int P, int NW, bool BOUNDS>
__global__ __launch_bounds__(64 * NW) void decode_seg_kernel(SegArgs a,
                                                             const uint16_t* __restrict__ vp,
                                                             float qscale, float* __restrict__ out,
                                                             float* __restrict__ lse) {
  // keys [cap_keys + kSelectExtraWords], then the physical page of every entry [cap_keys]
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ int32_t sel_l[kMaxPagesPerSplit];
  __shared__ int32_t cnt_l;
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];
  __shared__ MfmaShared<G, NW> sm;
  static_assert(kMaxPagesPerSplit <= 64 * NW, "one page-list entry per thread");

  const int seg = blockIdx.x;
  int* pid_l = (int*)(dyn + a.cap_keys + kSelectExtraWords);
  index_segment<uint16_t, uint16_t, 128, G, NW, BOUNDS>(a, seg, dyn, pid_l, sel_l, &cnt_l);

  const Meta& m = a.m;
  const int b = seg / a.hkv, g = seg % a.hkv;
  u32x4 qa[4];
  mfma_load_q<G>((const uint16_t*)a.q, b, g, a.hkv, qa);
  __syncthreads();  // selection and page ids visible to the block
  const int count = min(cnt_l, kMaxPagesPerSplit);
  const int L = seq_len_clamped(m, b);
  if ((int)threadIdx.x < count) {
    const int lp = sel_l[threadIdx.x];
    pg_phys[threadIdx.x] = pid_l[lp];
    pg_nv[threadIdx.x] = max(0, min(P, L - lp * P));
  }
  __syncthreads();  // page list ready
  mfma_attend<G, P, NW>(sm, pg_phys, pg_nv, count, b, g, a.hkv, qa, (const uint16_t*)a.kp, vp,
                        qscale, 1, 0, out, lse, nullptr, nullptr);
}

template <typename KV, int G, int DK, int P, bool BOUNDS>
__global__ __launch_bounds__(64 * kVecWaves) void decode_seg_vec_kernel(SegArgs a,
                                                                    const KV* __restrict__ vp,
                                                                    float qscale,
                                                                    float* __restrict__ out,
                                                                    float* __restrict__ lse) {
  // keys [cap_keys + kSelectExtraWords], then the physical page of every entry [cap_keys]
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ int32_t sel_l[kMaxPagesPerSplit];
  __shared__ int32_t cnt_l;
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];
  __shared__ VecShared<G, DK> sm;
  static_assert(kMaxPagesPerSplit <= 64 * kVecWaves, "one page-list entry per thread");

  const int seg = blockIdx.x;
  int* pid_l = (int*)(dyn + a.cap_keys + kSelectExtraWords);
  index_segment<KV, KV, DK, G, kVecWaves, BOUNDS>(a, seg, dyn, pid_l, sel_l, &cnt_l);

  const Meta& m = a.m;
  const int b = seg / a.hkv, g = seg % a.hkv;
  VecQuery<KV, KV, G> vq;
  vec_load_q<KV, KV, G, DK>((const KV*)a.q, b, g, a.hkv, qscale, vq);
  __syncthreads();  // selection and page ids visible to the block
  const int count = min(cnt_l, kMaxPagesPerSplit);
  const int L = seq_len_clamped(m, b);
  if ((int)threadIdx.x < count) {
    const int lp = sel_l[threadIdx.x];
    pg_phys[threadIdx.x] = pid_l[lp];
    pg_nv[threadIdx.x] = max(0, min(P, L - lp * P));
  }
  __syncthreads();  // page list ready
  vec_attend<KV, KV, G, DK, P>(sm, pg_phys, pg_nv, count, b, g, a.hkv, vq, (const KV*)a.kp, vp,
                               qscale, 1, 0, out, lse, nullptr, nullptr);
}

template <typename KV, int DK, int P, bool BOUNDS>
hipError_t launch_vec(const SegArgs& a, const void* v_pool, float qscale, float* out, float* lse,
                      hipStream_t s) {
  dim3 grid(a.m.batch * a.hkv), block(64 * kVecWaves);
  const size_t lds = (size_t)(2 * a.cap_keys + kSelectExtraWords) * sizeof(uint32_t);
#define VX_VEC(GG)                                                                              \
  case GG:                                                                                      \
    hipLaunchKernelGGL((decode_seg_vec_kernel<KV, GG, DK, P, BOUNDS>), grid, block, lds, s, a, \
                       (const KV*)v_pool, qscale, out, lse);                                    \
    break;
  switch (a.hq / a.hkv) {
    VX_VEC(1)
    VX_VEC(2)
    VX_VEC(4)
    VX_VEC(8)
    default:
      return hipErrorInvalidValue;
  }
#undef VX_VEC
  return hipGetLastError();
}

template <int P>
hipError_t launch_vec_p(const SegArgs& a, const vx_geom& g, bool bounds, const void* v_pool,
                        float qscale, float* out, float* lse, hipStream_t s) {
  if (g.kv_dtype == VX_F32) {  // the bounds indexer is bf16 only (see decode_step_fusable)
    if (g.head_dim_k == 128) return launch_vec<float, 128, P, false>(a, v_pool, qscale, out, lse, s);
    return launch_vec<float, 64, P, false>(a, v_pool, qscale, out, lse, s);
  }
  if (bounds) return launch_vec<uint16_t, 64, P, true>(a, v_pool, qscale, out, lse, s);
  return launch_vec<uint16_t, 64, P, false>(a, v_pool, qscale, out, lse, s);
}

template <int G, int P, bool BOUNDS>
hipError_t launch_g(const SegArgs& a, const void* v_pool, float qscale, float* out, float* lse,
                    int max_pages, hipStream_t s) {
  dim3 grid(a.m.batch * a.hkv);
  const size_t lds = (size_t)(2 * a.cap_keys + kSelectExtraWords) * sizeof(uint32_t);
  if constexpr (G <= 4) {
    if (gqa_attn_waves(G, max_pages) == 16) {
      hipLaunchKernelGGL((decode_seg_kernel<G, P, 16, BOUNDS>), grid, dim3(1024), lds, s, a,
                         (const uint16_t*)v_pool, qscale, out, lse);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_seg_kernel<G, P, 8, BOUNDS>), grid, dim3(512), lds, s, a,
                     (const uint16_t*)v_pool, qscale, out, lse);
  return hipGetLastError();
}

template <int P, bool BOUNDS>
hipError_t launch_p(const SegArgs& a, const void* v_pool, float qscale, float* out, float* lse,
                    int max_pages, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_g<1, P, BOUNDS>(a, v_pool, qscale, out, lse, max_pages, s);
    case 2: return launch_g<2, P, BOUNDS>(a, v_pool, qscale, out, lse, max_pages, s);
    case 4: return launch_g<4, P, BOUNDS>(a, v_pool, qscale, out, lse, max_pages, s);
    case 8: return launch_g<8, P, BOUNDS>(a, v_pool, qscale, out, lse, max_pages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_step_fusable(const vx_geom& g, int page_size, int max_pages, int sel_stride,
                         bool bounds) {
  const int G = g.num_q_heads / g.num_kv_heads;
  return !g.mla && g.q_dtype == g.kv_dtype && (g.head_dim_k == 64 || g.head_dim_k == 128) &&
         (G == 1 || G == 2 || G == 4 || G == 8) && (page_size == 16 || page_size == 64) &&
         max_pages <= kMaxFusedStepPages && sel_stride <= kMaxPagesPerSplit &&
         !(bounds && g.kv_dtype == VX_F32);
}

hipError_t launch_decode_step_gqa(const Meta& m, const vx_geom& g, const void* q,
                                  const void* k_pool, const void* v_pool, float* cent,
                                  uint16_t* cent_bf16, void* bounds, int refresh, float score_scale,
                                  float sm_scale, float* scores, int k, int n_sink, int n_local,
                                  int mode, const uint32_t* rnd, int32_t* sel, int stride,
                                  int32_t* sel_count, float* out, float* lse, int max_pages,
                                  hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  SegArgs a{};
  a.m = m;
  a.hq = g.num_q_heads;
  a.hkv = g.num_kv_heads;
  a.q = q;
  a.kp = k_pool;
  a.cent = cent;
  a.cent_bf16 = cent_bf16;
  a.bounds = bounds;
  a.refresh = refresh;
  a.scale = score_scale;
  a.scores = scores;
  a.k = k;
  a.n_sink = n_sink;
  a.n_local = n_local;
  a.mode = mode;
  a.rnd = rnd;
  a.sel = sel;
  a.stride = stride;
  a.sel_count = sel_count;
  a.cap_keys = (max_pages + 63) / 64 * 64;
  const float qscale = sm_scale * kLog2e;
  if (!(g.kv_dtype == VX_BF16 && g.head_dim_k == 128)) {
    if (m.page_size == 16)
      return launch_vec_p<16>(a, g, bounds != nullptr, v_pool, qscale, out, lse, s);
    return launch_vec_p<64>(a, g, bounds != nullptr, v_pool, qscale, out, lse, s);
  }
  if (bounds) {
    if (m.page_size == 16) return launch_p<16, true>(a, v_pool, qscale, out, lse, max_pages, s);
    return launch_p<64, true>(a, v_pool, qscale, out, lse, max_pages, s);
  }
  if (m.page_size == 16) return launch_p<16, false>(a, v_pool, qscale, out, lse, max_pages, s);
  return launch_p<64, false>(a, v_pool, qscale, out, lse, max_pages, s);
}

}  // namespace vx
