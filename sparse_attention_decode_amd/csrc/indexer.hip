// Indexer kernel, GQA geometry: one block per (sequence, KV head) segment
// runs index_segment (index_seg.h): newest-page refresh, scores, top-k.
#include "index_seg.h"

namespace vx {
namespace {

// Waves per block: 16 for short segments (more page loads in flight at
// once), 8 for long ones (a block's work then needs fewer waves, and more
// blocks fit a compute unit); the bound is kMaxSegPagesFor16.

// CB16: scores on the bf16 copy of the centroids (index_seg.h).
template <typename QT, typename KV, int DK, int GG, int NW, bool CB16>
__global__ __launch_bounds__(64 * NW) void index_seg_kernel(SegArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];  // cap_keys + kSelectExtraWords
  index_segment<QT, KV, DK, GG, NW, false, CB16>(a, blockIdx.x, keys, nullptr, nullptr, nullptr);
}

template <typename QT, typename KV, int DK, int NW, bool CB16>
hipError_t launch_nw(const SegArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  dim3 grid(a.m.batch * a.hkv), block(64 * NW);
  const size_t lds = (size_t)(a.cap_keys + kSelectExtraWords) * sizeof(uint32_t);
#define VX_SEG(GG) \
  hipLaunchKernelGGL((index_seg_kernel<QT, KV, DK, GG, NW, CB16>), grid, block, lds, s, a)
  switch (G) {
    case 1: VX_SEG(1); break;
    case 2: VX_SEG(2); break;
    case 4: VX_SEG(4); break;
    case 8: VX_SEG(8); break;
    default: VX_SEG(0); break;
  }
#undef VX_SEG
  return hipGetLastError();
}

template <typename QT, typename KV, int DK, bool CB16 = false>
hipError_t launch_dk(const SegArgs& a, int max_pages, hipStream_t s) {
  if (max_pages <= kMaxSegPagesFor16) return launch_nw<QT, KV, DK, 16, CB16>(a, s);
  return launch_nw<QT, KV, DK, 8, CB16>(a, s);
}

}  // namespace

hipError_t launch_index_gqa(const Meta& m, const vx_geom& g, const void* q, const void* k_pool,
                            float* cent, uint16_t* cent_bf16, int refresh, float scale,
                            float* scores, int k, int n_sink, int n_local, int mode,
                            const uint32_t* rnd, int32_t* sel, int stride, int32_t* sel_count,
                            int max_pages, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  SegArgs a{};
  a.m = m;
  a.hq = g.num_q_heads;
  a.hkv = g.num_kv_heads;
  a.q = q;
  a.kp = k_pool;
  a.cent = cent;
  a.cent_bf16 = cent_bf16;
  a.refresh = refresh;
  a.scale = scale;
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
  const bool f32 = g.kv_dtype == VX_F32;  // the bf16 copy is scored with bf16 keys only
  if (g.head_dim_k == 64)
    return f32 ? launch_dk<float, float, 64>(a, max_pages, s)
               : g.score_bf16 ? launch_dk<uint16_t, uint16_t, 64, true>(a, max_pages, s)
                              : launch_dk<uint16_t, uint16_t, 64>(a, max_pages, s);
  return f32 ? launch_dk<float, float, 128>(a, max_pages, s)
             : g.score_bf16 ? launch_dk<uint16_t, uint16_t, 128, true>(a, max_pages, s)
                            : launch_dk<uint16_t, uint16_t, 128>(a, max_pages, s);
}

}  // namespace vx
