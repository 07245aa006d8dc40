// Quest-style indexer, GQA geometry: per-page key bounds (cache stage) and
// their upper-bound page scores.
//
// Quest (Tang et al., "Quest: Query-Aware Sparsity for Efficient
// Long-Context LLM Inference", ICML 2024), the other baseline the Vortex
// paper note measures against ("Paper context", "Key results > User-side
// latency"), keeps per page the elementwise minimum and maximum of its keys
// and ranks pages by an upper bound of the query-key product:
//   score = scale * sum_d max(Q_d * lo_d, Q_d * hi_d),
// Q the group-summed query of the KV head (the query the centroid indexer
// uses), lo / hi the page's bounds. Selection and attention are the shared
// top-k and attention kernels.
//
// Bounds are stored in the KV dtype: the minimum and maximum of bf16 keys
// are bf16 values, so nothing is rounded and a page costs as many bytes as
// an fp32 centroid row. Layout [pool][Hkv][Dk/4][2][4]: for each group of 4
// dims, their 4 minima then their 4 maxima, so one 16-byte load (bf16) gives
// a lane both bounds of its dims and consecutive lanes read consecutive
// bytes.
//
// Scorer mapping: a flat grid over page-table entries, so no block idles
// past a short sequence's pages; every load instruction reads 1 KB of
// contiguous bounds (bf16). W = Dk / 4 lanes cover a KV head and reduce with
// DPP. A wave has several pages' rows in flight, issued as soon as their
// page ids arrive, while the block finds its first entry's sequence and sums
// that sequence's query into LDS once. With refresh on, one extra block per
// sequence recomputes the newest page's bounds from its keys, stores them
// and scores that page from the values it computed (same arithmetic as the
// other blocks); the other blocks skip that page. The whole-step kernel runs
// the same arithmetic per (sequence, KV head) segment (index_seg.h).
#include "bounds.h"

namespace vx {
namespace {

template <typename KV>
__global__ void bounds_rebuild_kernel(Meta m, int hkv, int dk, const KV* __restrict__ kp,
                                      KV* __restrict__ bounds) {
  const int j = blockIdx.x;
  if (j >= m.nnz) return;
  const int b = find_seq(m.indptr, m.batch, j);
  const int L = seq_len_clamped(m, b);
  const int p = j - m.indptr[b];
  int nv = L - p * m.page_size;
  nv = nv < 0 ? 0 : (nv > m.page_size ? m.page_size : nv);
  const int pid = phys_page(m, j);
  for (int u = threadIdx.x; u < hkv * dk / 4; u += blockDim.x) {
    float lo[4], hi[4];
    unit_bounds<KV>(kp, bounds, m.page_size, hkv, dk, pid, nv, u, lo, hi);
  }
}

template <typename KV>
__global__ void bounds_append_kernel(Meta m, int hkv, int dk, const KV* __restrict__ kp,
                                     const int32_t* __restrict__ first_token,
                                     KV* __restrict__ bounds) {
  const int b = blockIdx.x;
  if (b >= m.batch) return;
  const int L = seq_len_clamped(m, b);
  if (L <= 0) return;
  const int P = m.page_size;
  const int last = L - 1;
  int ft = first_token[b];
  if (ft < 0) ft += L;  // negative: counted from the end (-1 = newest token)
  ft = ft < 0 ? 0 : (ft > last ? last : ft);
  for (int p = ft / P; p <= last / P; ++p) {
    const int nv = min(P, L - p * P);
    const int pid = phys_page(m, m.indptr[b] + p);
    for (int u = threadIdx.x; u < hkv * dk / 4; u += blockDim.x) {
      float lo[4], hi[4];
      unit_bounds<KV>(kp, bounds, P, hkv, dk, pid, nv, u, lo, hi);
    }
  }
}

struct BoundArgs {
  Meta m;
  int hq, hkv;
  const void* q;
  const void* kp;     // key pool (refresh only)
  void* bounds;       // [pool][Hkv][Dk/4][2][4] in the KV dtype
  int refresh;
  float scale;
  float* scores;      // [Hkv][nnz]
  int ppw;            // entries per wave (scorer), at most its PPW
};

// Scaled group-summed query of sequence b, KV head g, dims d .. d+3: the
// group's heads added in head order in fp32, then the scale. GG > 0: the
// group size, known at compile time (all loads in flight at once).
template <typename QT, int DK, int GG>
VX_DEV float4 group_query4(const QT* __restrict__ q, int hq, int G, int b, int g, int d,
                           float scale) {
  const QT* qb = q + ((size_t)b * hq + (size_t)g * G) * DK + d;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (GG > 0) {
    typename Quad<QT>::raw x[GG];
#pragma unroll
    for (int h = 0; h < GG; ++h) x[h] = Quad<QT>::load(qb + (size_t)h * DK);
#pragma unroll
    for (int h = 0; h < GG; ++h) {
      const float4 v = Quad<QT>::widen(x[h]);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  } else {
    for (int h = 0; h < G; ++h) {
      const float4 v = Quad<QT>::widen(Quad<QT>::load(qb + (size_t)h * DK));
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  return make_float4(s.x * scale, s.y * scale, s.z * scale, s.w * scale);
}

constexpr int kScoreWaves = 8;
constexpr int kScoreThreads = 64 * kScoreWaves;  // >= C = Hkv * Dk / 4 (<= 512)

// Grid: ceil(nnz / (8 * ppw)) blocks of 8 waves over page-table entries,
// then (refresh) one block per sequence. A wave scores ppw <= PPW consecutive
// entries; lane l holds units c = i * 64 + l (i < R, c < C) of every row, so
// each load instruction reads 1 KB of contiguous bounds (bf16). Two chains
// run side by side: page ids -> rows, and the block's first entry's
// sequence (one ballot round) -> its query units, summed once per block
// into LDS, and a window of the next 63 sequences' table starts and lengths
// (lane i holds sequence b_blk + i's), from which one ballot gives any
// entry's sequence. An entry of another sequence than the block's first
// sums its own query units (uniform over the wave).
template <typename QT, typename KV, int DK, int R, int PPW, int GG>
__global__ __launch_bounds__(kScoreThreads) void bound_scores_kernel(BoundArgs a) {
  constexpr int W = DK / 4;  // lanes per KV head
  __shared__ float4 qsum[kScoreThreads];

  const Meta& m = a.m;
  const QT* q = (const QT*)a.q;
  KV* bounds = (KV*)a.bounds;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = GG > 0 ? GG : a.hq / a.hkv;
  const int P = m.page_size;
  const int C = a.hkv * W;
  const int ppw = a.ppw;
  const int nflat = (m.nnz + kScoreWaves * ppw - 1) / (kScoreWaves * ppw);
  const size_t nnz = (size_t)m.nnz;

  if ((int)blockIdx.x >= nflat) {
    // refresh block of sequence b: recompute, store and score its newest page
    const int b = blockIdx.x - nflat;
    const int L = seq_len_clamped(m, b);
    if (L == 0) return;
    const int p = (L - 1) / P;
    const int nv = L - p * P;
    const int j = m.indptr[b] + p;
    const int pid = phys_page(m, j);
    const int u = tid;  // C <= kScoreThreads
    const bool ok = u < C;
    float s = 0.f;
    if (ok) {
      float lo[4], hi[4];
      unit_bounds<KV>((const KV*)a.kp, bounds, P, a.hkv, DK, pid, nv, u, lo, hi);
      s = unit_bound(group_query4<QT, DK, GG>(q, a.hq, G, b, u / W, 4 * (u % W), a.scale), lo,
                     hi);
    }
    s = group_sum<W>(s);
    if (ok && (u % W) == 0) a.scores[(size_t)(u / W) * nnz + j] = s;
    return;
  }

  const int j_blk = blockIdx.x * kScoreWaves * ppw;
  const int jw = j_blk + w * ppw;  // the wave's first entry
  const int nj = max(0, min(ppw, m.nnz - jw));
  // chain 1: page ids (lane k loads entry jw + k's), then every row unit (an
  // entry past its sequence's pages in use is loaded for nothing)
  const int my_pid = nj > 0 ? phys_page(m, jw + min(lane, nj - 1)) : 0;
  typename Unit<KV>::raw raw[PPW][R];
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    if (k < nj) {
      const KV* row = bounds + (size_t)__builtin_amdgcn_readlane(my_pid, k) * C * 8;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = i * 64 + lane;
        if (c < C) raw[k][i] = Unit<KV>::load(row + (size_t)c * 8);
      }
    }
  }
  // chain 2: the block's first sequence and its query units
  const int b_blk = __builtin_amdgcn_readfirstlane(wave_find_seq(m.indptr, m.batch, j_blk, lane));
  if (tid < C)
    qsum[tid] = group_query4<QT, DK, GG>(q, a.hq, G, b_blk, tid / W, 4 * (tid % W), a.scale);
  const int wnd = m.indptr[min(b_blk + lane, m.batch)];
  const int wlen = m.seq_lens[min(b_blk + lane, m.batch - 1)];
  __syncthreads();

#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    if (k >= nj) break;
    const int j = jw + k;
    const int cb = __popcll(__ballot(lane >= 1 && wnd <= j));
    int b, s0, s1, L;
    if (cb < 63) {
      b = b_blk + cb;
      s0 = __builtin_amdgcn_readlane(wnd, cb);
      s1 = __builtin_amdgcn_readlane(wnd, cb + 1);
      L = __builtin_amdgcn_readlane(wlen, cb);
    } else {  // past a run of 62 sequences without entries
      b = __builtin_amdgcn_readfirstlane(wave_find_seq(m.indptr, m.batch, j, lane));
      s0 = m.indptr[b];
      s1 = m.indptr[b + 1];
      L = m.seq_lens[b];
    }
    L = min(max(L, 0), (s1 - s0) * P);
    const int n = (L + P - 1) / P;
    const int p = j - s0;
    const bool other = b != b_blk;
    const int n_scored = (a.refresh && n > 0) ? n - 1 : n;
    if (p >= n_scored) continue;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = i * 64 + lane;
      float s = 0.f;
      if (c < C) {
        float lo[4], hi[4];
        Unit<KV>::widen(raw[k][i], lo, hi);
        const float4 qk =
            other ? group_query4<QT, DK, GG>(q, a.hq, G, b, c / W, 4 * (c % W), a.scale)
                  : qsum[c];
        s = unit_bound(qk, lo, hi);
      }
      s = group_sum<W>(s);
      if (c < C && (c % W) == 0) a.scores[(size_t)(c / W) * nnz + j] = s;
    }
  }
}

// Entries per wave: up to PPW (16 rows in flight per lane for R >= 4),
// fewer while that leaves under two blocks per compute unit.
template <typename QT, typename KV, int DK, int R, int GG>
void launch_bound_scores_g(BoundArgs a, hipStream_t s) {
  constexpr int PPW = R >= 4 ? 16 / R : 4;
  int ppw = PPW;
  while (ppw > 1 && (long)a.m.nnz < 2L * 256 * kScoreWaves * ppw) ppw /= 2;
  a.ppw = ppw;
  const int per_block = kScoreWaves * ppw;
  const dim3 grid((unsigned)((a.m.nnz + per_block - 1) / per_block +
                             (a.refresh ? a.m.batch : 0)));
  hipLaunchKernelGGL((bound_scores_kernel<QT, KV, DK, R, PPW, GG>), grid, dim3(kScoreThreads), 0,
                     s, a);
}

template <typename QT, typename KV, int DK, int R>
void launch_bound_scores_r(const BoundArgs& a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: launch_bound_scores_g<QT, KV, DK, R, 1>(a, s); break;
    case 2: launch_bound_scores_g<QT, KV, DK, R, 2>(a, s); break;
    case 4: launch_bound_scores_g<QT, KV, DK, R, 4>(a, s); break;
    case 8: launch_bound_scores_g<QT, KV, DK, R, 8>(a, s); break;
    default: launch_bound_scores_g<QT, KV, DK, R, 0>(a, s); break;
  }
}

template <typename QT, typename KV, int DK>
void launch_bound_scores_t(const BoundArgs& a, int C, hipStream_t s) {
  const int r = (C + 63) / 64;  // <= 8
  if (r <= 1) launch_bound_scores_r<QT, KV, DK, 1>(a, s);
  else if (r <= 2) launch_bound_scores_r<QT, KV, DK, 2>(a, s);
  else if (r <= 4) launch_bound_scores_r<QT, KV, DK, 4>(a, s);
  else launch_bound_scores_r<QT, KV, DK, 8>(a, s);
}

int block_for_units(int units) {
  int t = ((units + 63) / 64) * 64;
  return t < 64 ? 64 : (t > 1024 ? 1024 : t);
}

}  // namespace

hipError_t launch_bounds_update(const Meta& m, const vx_geom& g, const void* k_pool,
                                const int32_t* first_token, void* bounds, hipStream_t s) {
  const int hkv = g.num_kv_heads, dk = g.head_dim_k;
  const dim3 block(block_for_units(hkv * dk / 4));
  if (!first_token) {
    if (m.nnz == 0) return hipSuccess;
    if (g.kv_dtype == VX_F32)
      hipLaunchKernelGGL(bounds_rebuild_kernel<float>, dim3(m.nnz), block, 0, s, m, hkv, dk,
                         (const float*)k_pool, (float*)bounds);
    else
      hipLaunchKernelGGL(bounds_rebuild_kernel<uint16_t>, dim3(m.nnz), block, 0, s, m, hkv, dk,
                         (const uint16_t*)k_pool, (uint16_t*)bounds);
  } else {
    if (m.batch == 0) return hipSuccess;
    if (g.kv_dtype == VX_F32)
      hipLaunchKernelGGL(bounds_append_kernel<float>, dim3(m.batch), block, 0, s, m, hkv, dk,
                         (const float*)k_pool, first_token, (float*)bounds);
    else
      hipLaunchKernelGGL(bounds_append_kernel<uint16_t>, dim3(m.batch), block, 0, s, m, hkv, dk,
                         (const uint16_t*)k_pool, first_token, (uint16_t*)bounds);
  }
  return hipGetLastError();
}

hipError_t launch_bound_scores(const Meta& m, const vx_geom& g, const void* q, const void* k_pool,
                               void* bounds, int refresh, float scale, float* scores,
                               int max_pages, hipStream_t s) {
  (void)max_pages;
  if (m.batch == 0 || m.nnz == 0) return hipSuccess;
  BoundArgs a;
  a.m = m;
  a.hq = g.num_q_heads;
  a.hkv = g.num_kv_heads;
  a.q = q;
  a.kp = k_pool;
  a.bounds = bounds;
  a.refresh = refresh;
  a.scale = scale;
  a.scores = scores;
  const bool f32 = g.kv_dtype == VX_F32;
  const int C = g.num_kv_heads * g.head_dim_k / 4;  // <= 512 by the geometry checks
  if (g.head_dim_k == 128) {
    if (f32) launch_bound_scores_t<float, float, 128>(a, C, s);
    else launch_bound_scores_t<uint16_t, uint16_t, 128>(a, C, s);
  } else {
    if (f32) launch_bound_scores_t<float, float, 64>(a, C, s);
    else launch_bound_scores_t<uint16_t, uint16_t, 64>(a, C, s);
  }
  return hipGetLastError();
}

}  // namespace vx
