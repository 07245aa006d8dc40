// Indexer scoring, GQA geometry: one fp32 GEMV per KV head over all pages.
//
// Vortex paper note, "System design > 1. vFlow": the indexer multiplies the
// query with the cached centroids. A GQA group's query heads share their KV
// head's pages, so the group's heads are summed first (by linearity the same
// score) and each page costs one dot product per KV head: the kernel streams
// every centroid row exactly once and is HBM bound (~0.5 flop/byte).
//
// Mapping: each wave owns `ppw` consecutive page-table entries. A centroid
// row [Hkv][Dk] fp32 is read as 16-byte chunks, chunk c = i*64 + lane, so
// every load instruction of a wave covers 1 KB contiguous. Chunk c belongs to
// head c / (Dk/4); the Dk/4 lanes of a head reduce with DPP row ops.
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kUnroll = 4;  // page rows in flight per wave

template <typename QT> struct QLoad;
template <> struct QLoad<float> {
  static __device__ __forceinline__ float4 get(const float* p) { return *(const float4*)p; }
};
template <> struct QLoad<uint16_t> {
  static __device__ __forceinline__ float4 get(const uint16_t* p) {
    uint2 w = *(const uint2*)p;
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  }
};

template <typename QT, int DK, int R>
__global__ __launch_bounds__(256) void scores_gqa_kernel(Meta m, int hq, int hkv,
                                                         const QT* __restrict__ q,
                                                         const float* __restrict__ cent,
                                                         float scale, float* __restrict__ scores,
                                                         int ppw) {
  constexpr int W = DK / 4;  // lanes per head row
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int j0 = wave * ppw;
  if (j0 >= m.nnz) return;
  const int j1 = min(j0 + ppw, m.nnz);
  const int nchunk = hkv * DK / 4;
  const int G = hq / hkv;
  const int rowlen = hkv * DK;

  int b = find_seq(m.indptr, m.batch, j0);
  int bstart = m.indptr[b], bend = m.indptr[b + 1];
  int npg = (seq_len_clamped(m, b) + m.page_size - 1) / m.page_size;

  float4 qs[R];
  auto load_q = [&](int bb) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = i * 64 + lane;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nchunk) {
        const int g = c / W, d = (c % W) * 4;
        const QT* qb = q + ((size_t)bb * hq + (size_t)g * G) * DK + d;
        for (int h = 0; h < G; ++h) {
          float4 x = QLoad<QT>::get(qb + (size_t)h * DK);
          a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
        }
        a.x *= scale; a.y *= scale; a.z *= scale; a.w *= scale;
      }
      qs[i] = a;
    }
  };
  int qseq = b;  // sequence whose group sums sit in qs
  load_q(qseq);

  for (int jb = j0; jb < j1; jb += kUnroll) {
    float4 c[kUnroll][R];
    int bj[kUnroll];
    bool ok[kUnroll];
    // Resolve the owning sequence of each entry and issue the row loads.
    int bb = b, bs = bstart, be = bend, np = npg;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = jb + u;
      ok[u] = false;
      bj[u] = bb;
      if (j < j1) {
        while (j >= be) {
          ++bb;
          bs = be;
          be = m.indptr[bb + 1];
          np = (seq_len_clamped(m, bb) + m.page_size - 1) / m.page_size;
        }
        bj[u] = bb;
        ok[u] = (j - bs) < np;
      }
      if (ok[u]) {
        const float* row = cent + (size_t)phys_page(m, j) * rowlen;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int ch = i * 64 + lane;
          c[u][i] = ch < nchunk ? *(const float4*)(row + 4 * ch) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!ok[u]) continue;
      if (bj[u] != qseq) {
        qseq = bj[u];
        load_q(qseq);
      }
      const int j = jb + u;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int ch = i * 64 + lane;
        float s = qs[i].x * c[u][i].x;
        s = fmaf(qs[i].y, c[u][i].y, s);
        s = fmaf(qs[i].z, c[u][i].z, s);
        s = fmaf(qs[i].w, c[u][i].w, s);
        s = group_sum<W>(s);
        if (ch < nchunk && (ch % W) == 0) scores[(size_t)(ch / W) * m.nnz + j] = s;
      }
    }
    b = bb;
    bstart = bs;
    bend = be;
    npg = np;
  }
}

template <typename QT, int DK>
hipError_t launch_dk(const Meta& m, const vx_geom& g, const void* q, const float* cent, float scale,
                     float* scores, int ppw, hipStream_t s) {
  const int nchunk = g.num_kv_heads * DK / 4;
  const int waves = (m.nnz + ppw - 1) / ppw;
  dim3 block(256), grid((waves + 3) / 4);
  const QT* qq = (const QT*)q;
  if (nchunk <= 64)
    hipLaunchKernelGGL((scores_gqa_kernel<QT, DK, 1>), grid, block, 0, s, m, g.num_q_heads,
                       g.num_kv_heads, qq, cent, scale, scores, ppw);
  else if (nchunk <= 128)
    hipLaunchKernelGGL((scores_gqa_kernel<QT, DK, 2>), grid, block, 0, s, m, g.num_q_heads,
                       g.num_kv_heads, qq, cent, scale, scores, ppw);
  else if (nchunk <= 256)
    hipLaunchKernelGGL((scores_gqa_kernel<QT, DK, 4>), grid, block, 0, s, m, g.num_q_heads,
                       g.num_kv_heads, qq, cent, scale, scores, ppw);
  else
    hipLaunchKernelGGL((scores_gqa_kernel<QT, DK, 8>), grid, block, 0, s, m, g.num_q_heads,
                       g.num_kv_heads, qq, cent, scale, scores, ppw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scores_gqa(const Meta& m, const vx_geom& g, const void* q, const float* cent,
                             float scale, float* scores, int ppw, hipStream_t s) {
  if (m.nnz == 0) return hipSuccess;
  const bool qf = g.q_dtype == VX_F32;
  if (g.head_dim_k == 64)
    return qf ? launch_dk<float, 64>(m, g, q, cent, scale, scores, ppw, s)
              : launch_dk<uint16_t, 64>(m, g, q, cent, scale, scores, ppw, s);
  return qf ? launch_dk<float, 128>(m, g, q, cent, scale, scores, ppw, s)
            : launch_dk<uint16_t, 128>(m, g, q, cent, scale, scores, ppw, s);
}

}  // namespace vx
