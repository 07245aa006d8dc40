// Cache stage: per-page key centroids.
//
// Vortex paper note ("Vortex: Efficient and Programmable Sparse Attention
// Serving for AI Agents"), section "System design > 1. vFlow": the cache stage
// keeps a query-independent statistic per block; for block top-k it is the
// key centroid. Here: the mean of the page's valid keys, summed in fp32 in
// token order and divided once (IEEE divide), so a page refreshed after an
// append equals a full rebuild bit for bit.
//
// Thread mapping: one block per page (rebuild) or per sequence (append); each
// thread owns two adjacent dims of one KV head and walks the page's tokens in
// order. Loads of one token row are contiguous across the threads of a head.
#include "vx_internal.h"

namespace vx {
namespace {

template <typename T> struct Pair;
template <> struct Pair<float> {
  using raw = float2;
  static __device__ __forceinline__ float2 load(const float* p) { return *(const float2*)p; }
  static __device__ __forceinline__ float2 widen(float2 w) { return w; }
  static __device__ __forceinline__ float2 get(const float* p) { return *(const float2*)p; }
  static __device__ __forceinline__ void put(float* p, float2 v) { *(float2*)p = v; }
};
template <> struct Pair<uint16_t> {
  using raw = uint32_t;  // two bf16
  static __device__ __forceinline__ uint32_t load(const uint16_t* p) { return *(const uint32_t*)p; }
  static __device__ __forceinline__ float2 widen(uint32_t w) {
    return make_float2(bf16_lo(w), bf16_hi(w));
  }
  static __device__ __forceinline__ float2 get(const uint16_t* p) { return widen(load(p)); }
  static __device__ __forceinline__ void put(uint16_t* p, float2 v) {
    uint32_t w = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    *(uint32_t*)p = w;
  }
};

// Recompute the centroid of one page for the dim pair owned by `pair`.
// `nv` valid tokens; if `slot` >= 0 that token's value comes from `fresh`
// (the just-appended key) instead of memory. Every token's load is issued
// in batches of 32 (bf16) or 16 (fp32) tokens before the batch is added; the
// sums still run in token order.
template <typename KV>
__device__ __forceinline__ void refresh_pair(const KV* __restrict__ kp, int P, int hkv, int dk,
                                             int pid, int nv, int pair, int slot, float2 fresh,
                                             float* __restrict__ cent,
                                             uint16_t* __restrict__ cent_bf16) {
  constexpr int kTok = sizeof(KV) == 2 ? 32 : 16;  // 32 raw registers either way
  const int g = pair / (dk / 2);
  const int d = 2 * (pair % (dk / 2));
  const KV* base = kp + ((size_t)pid * hkv + g) * (size_t)P * dk + d;
  float s0 = 0.f, s1 = 0.f;
  for (int t0 = 0; t0 < nv; t0 += kTok) {
    typename Pair<KV>::raw x[kTok];
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int t = t0 + u;
      if (t < nv) x[u] = Pair<KV>::load(base + (size_t)t * dk);
    }
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int t = t0 + u;
      if (t < nv) {
        const float2 v = (t == slot) ? fresh : Pair<KV>::widen(x[u]);
        s0 += v.x;
        s1 += v.y;
      }
    }
  }
  float2 c = make_float2(0.f, 0.f);
  if (nv > 0) {
    c.x = s0 / (float)nv;
    c.y = s1 / (float)nv;
  }
  const size_t o = ((size_t)pid * hkv + g) * dk + d;
  Pair<float>::put(cent + o, c);
  if (cent_bf16) Pair<uint16_t>::put(cent_bf16 + o, c);
}

template <typename KV>
__global__ void centroid_rebuild_kernel(Meta m, int hkv, int dk, const KV* __restrict__ kp,
                                        float* __restrict__ cent, uint16_t* __restrict__ cent_bf16) {
  const int j = blockIdx.x;
  if (j >= m.nnz) return;
  const int b = find_seq(m.indptr, m.batch, j);
  const int L = seq_len_clamped(m, b);
  const int p = j - m.indptr[b];
  int nv = L - p * m.page_size;
  nv = nv < 0 ? 0 : (nv > m.page_size ? m.page_size : nv);
  const int pid = phys_page(m, j);
  const int pairs = hkv * dk / 2;
  for (int pr = threadIdx.x; pr < pairs; pr += blockDim.x)
    refresh_pair<KV>(kp, m.page_size, hkv, dk, pid, nv, pr, -1, make_float2(0.f, 0.f), cent,
                     cent_bf16);
}

template <typename KV>
__global__ void centroid_append_kernel(Meta m, int hkv, int dk, int dv, KV* __restrict__ kp,
                                       KV* __restrict__ vp, const int32_t* __restrict__ first_token,
                                       const KV* __restrict__ k_new, const KV* __restrict__ v_new,
                                       float* __restrict__ cent, uint16_t* __restrict__ cent_bf16) {
  const int b = blockIdx.x;
  if (b >= m.batch) return;
  const int L = seq_len_clamped(m, b);
  if (L <= 0) return;
  const int P = m.page_size;
  const int row0 = m.indptr[b];
  const int last = L - 1;
  const int last_page = last / P;
  const int last_slot = last % P;
  const int last_pid = phys_page(m, row0 + last_page);
  const int pairs = hkv * dk / 2;

  // Optional write of the newest token's K/V into its slot.
  if (v_new && vp) {
    for (int pr = threadIdx.x; pr < hkv * dv / 2; pr += blockDim.x) {
      const int g = pr / (dv / 2), d = 2 * (pr % (dv / 2));
      KV* dst = vp + (((size_t)last_pid * hkv + g) * P + last_slot) * dv + d;
      Pair<KV>::put(dst, Pair<KV>::get(v_new + ((size_t)b * hkv + g) * dv + d));
    }
  }

  int ft = first_token ? first_token[b] : -1;  // NULL: the newest token's page only
  if (ft < 0) ft += L;  // negative: counted from the end (-1 = newest token)
  ft = ft < 0 ? 0 : (ft > last ? last : ft);
  for (int p = ft / P; p <= last_page; ++p) {
    int nv = L - p * P;
    nv = nv > P ? P : nv;
    const int pid = phys_page(m, row0 + p);
    for (int pr = threadIdx.x; pr < pairs; pr += blockDim.x) {
      int slot = -1;
      float2 fresh = make_float2(0.f, 0.f);
      if (k_new && p == last_page) {
        const int g = pr / (dk / 2), d = 2 * (pr % (dk / 2));
        fresh = Pair<KV>::get(k_new + ((size_t)b * hkv + g) * dk + d);
        slot = last_slot;
        KV* dst = kp + (((size_t)pid * hkv + g) * P + last_slot) * dk + d;
        Pair<KV>::put(dst, fresh);
      }
      refresh_pair<KV>(kp, P, hkv, dk, pid, nv, pr, slot, fresh, cent, cent_bf16);
    }
  }
}

int block_for_pairs(int pairs) {
  int t = ((pairs + 63) / 64) * 64;
  return t < 64 ? 64 : (t > 1024 ? 1024 : t);
}

}  // namespace

hipError_t launch_centroid_rebuild(const Meta& m, const vx_geom& g, const void* k_pool,
                                   float* cent, uint16_t* cent_bf16, hipStream_t s) {
  if (m.nnz == 0) return hipSuccess;
  const int hkv = g.num_kv_heads, dk = g.head_dim_k;
  dim3 grid(m.nnz), block(block_for_pairs(hkv * dk / 2));
  if (g.kv_dtype == VX_F32)
    hipLaunchKernelGGL(centroid_rebuild_kernel<float>, grid, block, 0, s, m, hkv, dk,
                       (const float*)k_pool, cent, cent_bf16);
  else
    hipLaunchKernelGGL(centroid_rebuild_kernel<uint16_t>, grid, block, 0, s, m, hkv, dk,
                       (const uint16_t*)k_pool, cent, cent_bf16);
  return hipGetLastError();
}

hipError_t launch_centroid_append(const Meta& m, const vx_geom& g, void* k_pool, void* v_pool,
                                  const int32_t* first_token, const void* k_new,
                                  const void* v_new, float* cent, uint16_t* cent_bf16,
                                  hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  const int hkv = g.num_kv_heads, dk = g.head_dim_k, dv = g.head_dim_v;
  dim3 grid(m.batch), block(block_for_pairs(hkv * dk / 2));
  if (g.kv_dtype == VX_F32)
    hipLaunchKernelGGL(centroid_append_kernel<float>, grid, block, 0, s, m, hkv, dk, dv,
                       (float*)k_pool, (float*)v_pool, first_token, (const float*)k_new,
                       (const float*)v_new, cent, cent_bf16);
  else
    hipLaunchKernelGGL(centroid_append_kernel<uint16_t>, grid, block, 0, s, m, hkv, dk, dv,
                       (uint16_t*)k_pool, (uint16_t*)v_pool, first_token,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, cent, cent_bf16);
  return hipGetLastError();
}

}  // namespace vx
