// Device-side check of the paged metadata (the page-index structure of a
// vTensor: Vortex paper note, "System design > 2. vTensor"). The kernels
// assume a well-formed page table and only clamp what would leave a buffer;
// this kernel counts the violations so that a caller can find a corrupted
// table without reading it back to the host.
#include "vx_internal.h"

namespace vx {
namespace {

// One block. counts[0]: indptr out of order (indptr[0] != 0, a decrease,
// indptr[B] != nnz); counts[1]: sequences whose length lies outside
// [0, capacity * page_size] or whose capacity exceeds max_pages; counts[2]:
// page-table entries outside [0, pool). Reads indptr[0..B], seq_lens[0..B)
// and page_ids[0..nnz) only, never through a value it checks.
__global__ __launch_bounds__(1024) void check_pages_kernel(Meta m, int max_pages,
                                                           int32_t* __restrict__ counts) {
  __shared__ int c[3];
  const int t = threadIdx.x;
  if (t < 3) c[t] = 0;
  __syncthreads();
  int order = 0, lens = 0, ids = 0;
  if (m.batch > 0) {
    for (int b = t; b <= m.batch; b += blockDim.x) {
      const int v = m.indptr[b];
      order += (b == 0 ? v != 0 : v < m.indptr[b - 1]) ? 1 : 0;
      order += (b == m.batch && v != m.nnz) ? 1 : 0;
      if (b < m.batch) {
        const long cap = (long)m.indptr[b + 1] - v;
        const long L = m.seq_lens[b];
        lens += (L < 0 || L > cap * m.page_size || cap > max_pages) ? 1 : 0;
      }
    }
  }
  for (int j = t; j < m.nnz; j += blockDim.x) {
    const int p = m.page_ids[j];
    ids += (p < 0 || p >= m.pool) ? 1 : 0;
  }
  if (order) atomicAdd(&c[0], order);
  if (lens) atomicAdd(&c[1], lens);
  if (ids) atomicAdd(&c[2], ids);
  __syncthreads();
  if (t < 3) counts[t] = c[t];
}

}  // namespace

hipError_t launch_check_pages(const Meta& m, int max_pages, int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(check_pages_kernel, dim3(1), dim3(1024), 0, s, m, max_pages, counts);
  return hipGetLastError();
}

}  // namespace vx
