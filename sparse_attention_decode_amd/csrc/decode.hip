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
// place of the centroids; CB16: the centroids' bf16 copy scored in place of
// the fp32 rows (index_seg.h). bf16 keys with Dk = 128 attend on the matrix cores
// (mfma_attend); fp32 keys or Dk = 64 on the vector ALUs (vec_attend), the
// bodies of the stand-alone attention kernels, so the bits are the same.
#include "attn_mfma.h"
#include "attn_vec.h"
#include "index_seg.h"

namespace vx {
namespace {

// The segment (sequence b, KV head g) = b * Hkv + g this block serves: block
// row i = blockIdx.x / Hkv takes sequence order[i] when the planner ordered
// the sequences (longest first), else sequence i.
// With pair_rows = R: the sequences ranked by pages in use (most first,
// ties: lower index first; the same count the index uses), rows i < R take
// ranks 0 .. R - 1 and row R + k, which shares compute units with row k,
// rank B - 1 - k: each compute unit then holds one long and one short
// segment. Any order gives the same results (each segment is one block's
// whole work); this one balances the compute units. Every thread calls it
// (one barrier); counts: LDS, batch + 1 ints, free until the index phase.
VX_DEV int paired_row(const SegArgs& a, int* counts, int* row) {
  const Meta& m = a.m;
  const int B = m.batch, P = m.page_size;
  const int i = blockIdx.x / a.hkv;
  const int want = i < a.pair_rows ? i : B - 1 - (i - a.pair_rows);
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int cap = m.indptr[b + 1] - m.indptr[b];
    const int L = min(max(m.seq_lens[b], 0), cap * P);
    counts[b] = min((L + P - 1) / P, cap);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int nb = counts[b];
    int r = 0;
    for (int j = 0; j < B; ++j) {
      const int nj = counts[j];
      r += (nj > nb || (nj == nb && j < b)) ? 1 : 0;
    }
    if (r == want) *row = b;
  }
  __syncthreads();
  return *row;
}

__device__ __forceinline__ int block_segment(const SegArgs& a, int* counts, int* row) {
  const int i = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  if (a.pair_rows > 0) return paired_row(a, counts, row) * a.hkv + g;
  if (!a.order) return blockIdx.x;
  const int b = a.order[i];
  return (b < 0 ? 0 : (b >= a.m.batch ? a.m.batch - 1 : b)) * a.hkv + g;
}

// Sequences ranked by pages in use, most first (ties: lower index first):
// order[r] = the sequence of rank r, so the whole-step blocks that the GPU
// dispatches first take the longest segments and the last ones the
// shortest (the workload planning of the Vortex paper note, "System design >
// 3. Execution backend": plan by batch size and sequence length). One block,
// batch <= kMaxOrderedBatch.
__global__ __launch_bounds__(1024) void rank_sequences_kernel(Meta m, int32_t* __restrict__ order) {
  __shared__ int npg[kMaxOrderedBatch];
  for (int b = threadIdx.x; b < m.batch; b += blockDim.x) {
    const int cap = m.indptr[b + 1] - m.indptr[b];
    const int L = seq_len_clamped(m, b);
    npg[b] = min((L + m.page_size - 1) / m.page_size, cap);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < m.batch; b += blockDim.x) {
    const int nb = npg[b];
    int r = 0;
    for (int j = 0; j < m.batch; ++j) {
      const int nj = npg[j];
      r += (nj > nb || (nj == nb && j < b)) ? 1 : 0;
    }
    order[r] = b;
  }
}

// The whole-step kernels' selection (kept in LDS, count <= stride entries)
// to a.sel / a.sel_count, -1 past the count, by wave 0. The LDS copy stays
// unchanged from the select to here.
VX_DEV void write_selection(const SegArgs& a, int seg, const int32_t* sel_l, int count) {
  if (threadIdx.x >= 64) return;
  int32_t* so = a.sel + (size_t)seg * a.stride;
  for (int i = threadIdx.x; i < a.stride; i += 64) so[i] = i < count ? sel_l[i] : -1;
  if (threadIdx.x == 0) a.sel_count[seg] = count;
}

template <int G, int P, int NW, bool BOUNDS, bool CB16>
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
  __shared__ int row_l;

  const int seg = block_segment(a, (int*)dyn, &row_l);
  const int b = seg / a.hkv, g = seg % a.hkv;
  const uint16_t* kp = (const uint16_t*)a.kp;
  int* pid_l = (int*)(dyn + a.cap_keys + kSelectExtraWords);
  u32x4 qa[4];
  MfmaState st;
  st.init();
  // With a forced sink and newest page, the first and last page of the
  // selection are pages 0 and n-1 whatever the scores: while wave 0 selects,
  // the waves that the chunk deal gives their chunks attend them. Wave 0
  // loads its query rows before it selects, so that load is not waited for
  // at the barrier after the selection.
  bool q_loaded = false, ends_done = false;
  auto idle = [&](int n, int L, bool selects) {
    mfma_load_q<G>((const uint16_t*)a.q, b, g, a.hkv, qa);
    q_loaded = true;
    if (!selects && a.n_sink >= 1 && a.n_local >= 1 && n >= 1) {
      const ChunkDeal<P / 16> d(n >= 2 ? 2 : 1);
      mfma_end_chunks<G, P, NW>(sm, st, d, pid_l[0], min(P, L), pid_l[n - 1],
                                min(P, L - (n - 1) * P), g, a.hkv, qa, kp, vp, qscale);
      ends_done = true;
    }
  };
  // The selection goes to a.sel after the attention (write_selection), so
  // its stores are not waited for at the barriers in between.
  index_segment<uint16_t, uint16_t, 128, G, NW, BOUNDS, CB16>(a, seg, dyn, pid_l, sel_l, &cnt_l,
                                                              idle, false);

  const Meta& m = a.m;
  if (!q_loaded) mfma_load_q<G>((const uint16_t*)a.q, b, g, a.hkv, qa);
  __syncthreads();  // selection and page ids visible to the block
  const int count = min(cnt_l, kMaxPagesPerSplit);
  const int L = seq_len_clamped(m, b);
  if ((int)threadIdx.x < count) {
    const int lp = sel_l[threadIdx.x];
    pg_phys[threadIdx.x] = pid_l[lp];
    pg_nv[threadIdx.x] = max(0, min(P, L - lp * P));
  }
  __syncthreads();  // page list ready
  const ChunkDeal<P / 16> d(count);
  if (!ends_done && count > 0)
    mfma_end_chunks<G, P, NW>(sm, st, d, pg_phys[0], pg_nv[0], pg_phys[count - 1],
                              pg_nv[count - 1], g, a.hkv, qa, kp, vp, qscale);
  mfma_mid_chunks<G, P, NW>(sm, st, d, pg_phys, pg_nv, g, a.hkv, qa, kp, vp, qscale);
  mfma_finish<G, NW>(sm, st, b, g, a.hkv, 1, 0, out, lse, nullptr, nullptr);
  write_selection(a, seg, sel_l, count);
}

template <typename KV, int G, int DK, int P, bool BOUNDS, bool CB16>
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
  __shared__ int row_l;

  const int seg = block_segment(a, (int*)dyn, &row_l);
  int* pid_l = (int*)(dyn + a.cap_keys + kSelectExtraWords);
  index_segment<KV, KV, DK, G, kVecWaves, BOUNDS, CB16>(a, seg, dyn, pid_l, sel_l, &cnt_l,
                                                        NoIdle{}, false);

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
  write_selection(a, seg, sel_l, count);
}

template <typename KV, int DK, int P, bool BOUNDS, bool CB16>
hipError_t launch_vec(const SegArgs& a, const void* v_pool, float qscale, float* out, float* lse,
                      hipStream_t s) {
  dim3 grid(a.m.batch * a.hkv), block(64 * kVecWaves);
  const size_t lds = (size_t)(2 * a.cap_keys + kSelectExtraWords) * sizeof(uint32_t);
#define VX_VEC(GG)                                                                              \
  case GG:                                                                                      \
    hipLaunchKernelGGL((decode_seg_vec_kernel<KV, GG, DK, P, BOUNDS, CB16>), grid, block, lds, s, a, \
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
  // the bounds indexer and the bf16 centroid copy are bf16 only (host checks)
  if (g.kv_dtype == VX_F32) {
    if (g.head_dim_k == 128)
      return launch_vec<float, 128, P, false, false>(a, v_pool, qscale, out, lse, s);
    return launch_vec<float, 64, P, false, false>(a, v_pool, qscale, out, lse, s);
  }
  if (bounds) return launch_vec<uint16_t, 64, P, true, false>(a, v_pool, qscale, out, lse, s);
  if (g.score_bf16)
    return launch_vec<uint16_t, 64, P, false, true>(a, v_pool, qscale, out, lse, s);
  return launch_vec<uint16_t, 64, P, false, false>(a, v_pool, qscale, out, lse, s);
}

template <int G, int P, bool BOUNDS, bool CB16>
hipError_t launch_g(const SegArgs& a, const void* v_pool, float qscale, float* out, float* lse,
                    int max_pages, hipStream_t s) {
  dim3 grid(a.m.batch * a.hkv);
  const size_t lds = (size_t)(2 * a.cap_keys + kSelectExtraWords) * sizeof(uint32_t);
  if constexpr (G <= 4) {
    if (gqa_attn_waves(G, max_pages) == 16) {
      hipLaunchKernelGGL((decode_seg_kernel<G, P, 16, BOUNDS, CB16>), grid, dim3(1024), lds, s, a,
                         (const uint16_t*)v_pool, qscale, out, lse);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_seg_kernel<G, P, 8, BOUNDS, CB16>), grid, dim3(512), lds, s, a,
                     (const uint16_t*)v_pool, qscale, out, lse);
  return hipGetLastError();
}

template <int P, bool BOUNDS, bool CB16>
hipError_t launch_p(const SegArgs& a, const void* v_pool, float qscale, float* out, float* lse,
                    int max_pages, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_g<1, P, BOUNDS, CB16>(a, v_pool, qscale, out, lse, max_pages, s);
    case 2: return launch_g<2, P, BOUNDS, CB16>(a, v_pool, qscale, out, lse, max_pages, s);
    case 4: return launch_g<4, P, BOUNDS, CB16>(a, v_pool, qscale, out, lse, max_pages, s);
    case 8: return launch_g<8, P, BOUNDS, CB16>(a, v_pool, qscale, out, lse, max_pages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rank_sequences(const Meta& m, int32_t* order, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  if (m.batch > kMaxOrderedBatch) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rank_sequences_kernel, dim3(1), dim3(1024), 0, s, m, order);
  return hipGetLastError();
}

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
                                  const int32_t* order, int pair_rows, const void* k_new,
                                  const void* v_new, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  SegArgs a{};
  a.order = order;
  a.pair_rows = pair_rows;
  a.k_new = k_new;
  a.v_new = v_new;
  a.vp = const_cast<void*>(v_pool);
  a.dv = g.head_dim_v;
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
    if (m.page_size == 16)
      return launch_p<16, true, false>(a, v_pool, qscale, out, lse, max_pages, s);
    return launch_p<64, true, false>(a, v_pool, qscale, out, lse, max_pages, s);
  }
  if (g.score_bf16) {
    if (m.page_size == 16)
      return launch_p<16, false, true>(a, v_pool, qscale, out, lse, max_pages, s);
    return launch_p<64, false, true>(a, v_pool, qscale, out, lse, max_pages, s);
  }
  if (m.page_size == 16)
    return launch_p<16, false, false>(a, v_pool, qscale, out, lse, max_pages, s);
  return launch_p<64, false, false>(a, v_pool, qscale, out, lse, max_pages, s);
}

}  // namespace vx
