// Indexer selection kernels: one wave per (sequence, KV head) segment for
// short segments, one block per segment for long ones; the selection itself
// (radix top-k, exact or approximate) is in topk_wave.h, shared with the
// fused indexer.
#include "topk_wave.h"


namespace vx {
namespace {

__global__ __launch_bounds__(256) void topk_kernel(Meta m, int hkv, const float* __restrict__ scores,
                                                   int k, int n_sink, int n_local, int mode,
                                                   const uint32_t* __restrict__ rnd,
                                                   int32_t* __restrict__ sel, int stride,
                                                   int32_t* __restrict__ sel_count, int cap_keys) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int seg = blockIdx.x * (blockDim.x >> 6) + w;
  if (seg >= m.batch * hkv) return;  // whole wave; no block barrier below
  uint32_t* keys = lds + w * cap_keys;
  const int b = seg / hkv, g = seg % hkv;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  int n = (seq_len_clamped(m, b) + m.page_size - 1) / m.page_size;
  n = n > cap ? cap : n;
  wave_select(keys, cap_keys, scores + (size_t)g * m.nnz + row0, n, k, n_sink,
              n_local, mode, mode == VX_TOPK_APPROX ? rnd[seg] : 0u, sel + (size_t)seg * stride,
              stride, sel_count + seg, lane);
}

// Long segments: one block of kTopkBlockWaves waves per segment, all of
// them loading keys and building the digit histograms (block_select_keys).
constexpr int kTopkBlockWaves = 8;

__global__ __launch_bounds__(64 * kTopkBlockWaves) void topk_block_kernel(
    Meta m, int hkv, const float* __restrict__ scores, int k, int n_sink, int n_local, int mode,
    const uint32_t* __restrict__ rnd, int32_t* __restrict__ sel, int stride,
    int32_t* __restrict__ sel_count, int cap_keys) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];  // cap_keys + kSelectExtraWords
  const int seg = blockIdx.x;
  const int b = seg / hkv, g = seg % hkv;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  int n = (seq_len_clamped(m, b) + m.page_size - 1) / m.page_size;
  n = min(n > cap ? cap : n, cap_keys);
  const float* sc = scores + (size_t)g * m.nnz + row0;
  for (int i = threadIdx.x; i < n; i += 64 * kTopkBlockWaves)
    keys[i] = (i < n_sink || i >= n - n_local) ? 0u : topk_detail::score_key(sc[i]);
  __syncthreads();
  block_select_keys<kTopkBlockWaves>(keys, keys + cap_keys, keys + cap_keys + kSelectHistWords, n, k, n_sink,
                                     n_local, mode, mode == VX_TOPK_APPROX ? rnd[seg] : 0u,
                                     sel + (size_t)seg * stride, stride, sel_count + seg);
}

}  // namespace

hipError_t launch_topk_sized(const Meta& m, int hkv, const float* scores, int k, int n_sink,
                             int n_local, int mode, const uint32_t* rand_u32, int32_t* sel,
                             int sel_stride, int32_t* sel_count, int max_pages,
                             int waves_per_block, hipStream_t s) {
  const int segs = m.batch * hkv;
  if (segs == 0) return hipSuccess;
  const int cap_keys = ((max_pages + 63) / 64) * 64;
  if (max_pages > kBlockSelectMin) {
    const size_t lds = (size_t)(cap_keys + kSelectExtraWords) * sizeof(uint32_t);
    hipLaunchKernelGGL(topk_block_kernel, dim3(segs), dim3(64 * kTopkBlockWaves), lds, s, m, hkv,
                       scores, k, n_sink, n_local, mode, rand_u32, sel, sel_stride, sel_count,
                       cap_keys);
    return hipGetLastError();
  }
  const size_t lds = (size_t)waves_per_block * cap_keys * sizeof(uint32_t);
  dim3 block(64 * waves_per_block), grid((segs + waves_per_block - 1) / waves_per_block);
  hipLaunchKernelGGL(topk_kernel, grid, block, lds, s, m, hkv, scores, k, n_sink, n_local, mode,
                     rand_u32, sel, sel_stride, sel_count, cap_keys);
  return hipGetLastError();
}

}  // namespace vx
