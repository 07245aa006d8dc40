// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
// Nothing here is part of the public ABI (include/vx.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vx.h"

namespace vx {

// Launch-side copy of the paged metadata (passed to kernels by value).
struct Meta {
  int32_t batch;
  int32_t page_size;
  int32_t pool;
  int32_t nnz;
  const int32_t* indptr;
  const int32_t* page_ids;
  const int32_t* seq_lens;
};

// ---------------------------------------------------------------- device helpers
#if defined(__HIP_DEVICE_COMPILE__)
#define VX_DEV __device__ __forceinline__
#else
#define VX_DEV __device__ inline
#endif

VX_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
VX_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
VX_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs; NaN stays NaN).
VX_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sequence owning page-table entry j: largest b with indptr[b] <= j.
VX_DEV int find_seq(const int32_t* __restrict__ indptr, int batch, int j) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (indptr[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Sequence owning page-table entry j, computed by a whole wave: the number of
// sequences e in [1, batch) with indptr[e] <= j (indptr is non-decreasing, so
// that predicate holds on a prefix of e). A 256-ary search: each round every
// lane samples 4 evenly spaced entries of the remaining range and a ballot
// narrows it 256-fold, so batch <= 257 takes one round and <= 65537 two.
// Every lane returns the same value.
VX_DEV int wave_find_seq(const int32_t* __restrict__ indptr, int batch, int j, int lane) {
  int lo = 1, n = batch - 1;  // candidates e in [lo, lo + n); all e < lo hold
  while (n > 0) {
    const int step = (n + 255) / 256;
    int v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 64 * k + lane;
      v[k] = i * step < n ? indptr[lo + i * step] : 0x7fffffff;
    }
    int c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) c += __popcll(__ballot(v[k] <= j));
    if (c == 0) break;
    if (step == 1) return lo - 1 + c;
    const int nlo = lo + (c - 1) * step + 1;  // sample c-1 holds, sample c does not
    n = min(step - 1, lo + n - nlo);
    lo = nlo;
  }
  return lo - 1;
}

// Valid tokens of sequence b, clamped to its page-table capacity.
VX_DEV int seq_len_clamped(const Meta& m, int b) {
  int cap = (m.indptr[b + 1] - m.indptr[b]) * m.page_size;
  int L = m.seq_lens[b];
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// The dispatcher deals a launch's blocks to the chip's 8 XCDs (each with its
// own L2) round-robin by linear block id. xcd_major(i, n) renumbers the
// blocks [0, n) so that each XCD takes one contiguous run of the new ids:
// blocks that read the same rows (one sequence's query rows) then share an
// L2 instead of fetching them once per XCD. A bijection of [0, n).
constexpr int kXcds = 8;
VX_DEV int xcd_major(int i, int n) {
  const int per = n / kXcds, extra = n % kXcds, x = i % kXcds, j = i / kXcds;
  return x * per + (x < extra ? x : extra) + j;
}

VX_DEV int phys_page(const Meta& m, int j) {
  int p = m.page_ids[j];
  return p < 0 ? 0 : (p >= m.pool ? m.pool - 1 : p);
}

// DPP lane moves inside rows of 16 lanes.
template <int CTRL>
VX_DEV float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;  // row_ror:4
constexpr int DPP_ROR8 = 0x128;  // row_ror:8

// Sum over aligned groups of W lanes; every lane of the group gets the sum.
template <int W>
VX_DEV float group_sum(float x) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
  if constexpr (W >= 2) x += dpp<DPP_XOR1>(x);
  if constexpr (W >= 4) x += dpp<DPP_XOR2>(x);
  if constexpr (W == 8) x += __shfl_xor(x, 4);
  if constexpr (W >= 16) { x += dpp<DPP_ROR4>(x); x += dpp<DPP_ROR8>(x); }
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int W>
VX_DEV float group_max(float x) {
  if constexpr (W >= 2) x = fmaxf(x, dpp<DPP_XOR1>(x));
  if constexpr (W >= 4) x = fmaxf(x, dpp<DPP_XOR2>(x));
  if constexpr (W == 8) x = fmaxf(x, __shfl_xor(x, 4));
  if constexpr (W >= 16) { x = fmaxf(x, dpp<DPP_ROR4>(x)); x = fmaxf(x, dpp<DPP_ROR8>(x)); }
  if constexpr (W >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (W >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Softmax constants: logits are kept in log2 units (exp2 on the ALUs).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

// Log-sum-exp merge of S split partials of one (sequence, head), 4 value
// columns: po = partial outputs (split stride dv), ml = (m, l) pairs per
// split; out[0..3] = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - max m),
// *lse (nullable) = (max m + log2 sum_s w_s l_s) ln 2. Up to kMergeBatch splits
// have every load in flight at once; the arithmetic and its order are the
// same for any S (so every merge writes the same bits).
constexpr int kMergeBatch = 16;
typedef float f32x4v __attribute__((ext_vector_type(4)));
VX_DEV float4 load_nt4(const float* p) {  // a partial row: read once
  const f32x4v r = __builtin_nontemporal_load((const f32x4v*)p);
  return make_float4(r.x, r.y, r.z, r.w);
}
VX_DEV void merge_row(int S, int dv, const float* __restrict__ po, const float* __restrict__ ml,
                      float* __restrict__ out, float* __restrict__ lse) {
  float mmax = kNegBig;
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (S <= kMergeBatch) {
    float2 mlv[kMergeBatch];
    float4 x[kMergeBatch];
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s) {
      if (s < S) {
        mlv[s] = *(const float2*)(ml + 2 * s);
        x[s] = load_nt4(po + (size_t)s * dv);
      }
    }
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s)
      if (s < S) mmax = fmaxf(mmax, mlv[s].x);
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s) {
      if (s < S) {
        const float wt = __builtin_amdgcn_exp2f(mlv[s].x - mmax);
        wsum = fmaf(mlv[s].y, wt, wsum);
        acc.x = fmaf(x[s].x, wt, acc.x); acc.y = fmaf(x[s].y, wt, acc.y);
        acc.z = fmaf(x[s].z, wt, acc.z); acc.w = fmaf(x[s].w, wt, acc.w);
      }
    }
  } else {
    for (int s = 0; s < S; ++s) mmax = fmaxf(mmax, ml[2 * s]);
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
      const float wt = __builtin_amdgcn_exp2f(ml[2 * s] - mmax);
      wsum = fmaf(ml[2 * s + 1], wt, wsum);
      const float4 xs = load_nt4(po + (size_t)s * dv);
      acc.x = fmaf(xs.x, wt, acc.x); acc.y = fmaf(xs.y, wt, acc.y);
      acc.z = fmaf(xs.z, wt, acc.z); acc.w = fmaf(xs.w, wt, acc.w);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *(float4*)out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse) *lse = wsum > 0.f ? (mmax + log2f(wsum)) * kLn2 : -INFINITY;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive elements: raw load, then widening to fp32 (kept apart so
// that many loads can be in flight in raw form).
template <typename T> struct Quad;
template <> struct Quad<float> {
  using raw = float4;
  static VX_DEV float4 load(const float* p) { return *(const float4*)p; }
  static VX_DEV float4 widen(float4 r) { return r; }
};
template <> struct Quad<uint16_t> {
  using raw = uint2;
  static VX_DEV uint2 load(const uint16_t* p) { return *(const uint2*)p; }
  static VX_DEV float4 widen(uint2 w) {
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  }
};

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. Shapes are validated by the
// caller (vx_capi.hip) before these run.

hipError_t launch_centroid_rebuild(const Meta& m, const vx_geom& g, const void* k_pool,
                                   float* cent, uint16_t* cent_bf16, hipStream_t s);
hipError_t launch_centroid_append(const Meta& m, const vx_geom& g, void* k_pool, void* v_pool,
                                  const int32_t* first_token, const void* k_new,
                                  const void* v_new, float* cent, uint16_t* cent_bf16,
                                  hipStream_t s);
// GQA scores; refresh != 0 first recomputes the centroid (and its bf16 copy
// when cent_bf16 is given) of each sequence's newest page, reading k_pool.
hipError_t launch_scores_gqa(const Meta& m, const vx_geom& g, const void* q, const void* k_pool,
                             float* cent, uint16_t* cent_bf16, int refresh, float scale,
                             float* scores, hipStream_t s);
// Fused GQA indexer, one block per (sequence, KV head): newest-page refresh
// (optional), scores and the top-k selection.
hipError_t launch_index_gqa(const Meta& m, const vx_geom& g, const void* q, const void* k_pool,
                            float* cent, uint16_t* cent_bf16, int refresh, float scale,
                            float* scores, int k, int n_sink, int n_local, int mode,
                            const uint32_t* rnd, int32_t* sel, int stride, int32_t* sel_count,
                            int max_pages, hipStream_t s);
// Whole step per (sequence, KV head) in one kernel (GQA, one split):
// index_segment then mfma_attend (bf16, Dk = 128) or vec_attend (fp32 keys or
// Dk = 64). bounds != NULL: the Quest-style indexer on those page bounds
// (cent and cent_bf16 unused; bf16 keys only).
bool decode_step_fusable(const vx_geom& g, int page_size, int max_pages, int sel_stride,
                         bool bounds);
hipError_t launch_decode_step_gqa(const Meta& m, const vx_geom& g, const void* q,
                                  const void* k_pool, const void* v_pool, float* cent,
                                  uint16_t* cent_bf16, void* bounds, int refresh, float score_scale,
                                  float sm_scale, float* scores, int k, int n_sink, int n_local,
                                  int mode, const uint32_t* rnd, int32_t* sel, int stride,
                                  int32_t* sel_count, float* out, float* lse, int max_pages,
                                  const int32_t* order, int pair_rows, const void* k_new,
                                  const void* v_new, hipStream_t s);
// order[r] = the sequence with the r-th most pages in use (ties: lower index
// first), for the whole-step kernel's block order. batch <= kMaxOrderedBatch.
hipError_t launch_rank_sequences(const Meta& m, int32_t* order, hipStream_t s);
// counts[0..3) = violations of the page-table contract (vx_check_pages).
hipError_t launch_check_pages(const Meta& m, int max_pages, int32_t* counts, hipStream_t s);
// MLA scores on the bf16 centroids; refresh != 0 first recomputes each
// sequence's newest page (fp32 centroid and its bf16 copy) from k_pool.
hipError_t launch_scores_mla_sized(const Meta& m, const vx_geom& g, const void* q,
                                   const void* k_pool, float* cent32, uint16_t* cent_bf16,
                                   int refresh, float scale, float* scores, int max_pages,
                                   hipStream_t s);
hipError_t launch_topk_sized(const Meta& m, int hkv, const float* scores, int k, int n_sink,
                             int n_local, int mode, const uint32_t* rand_u32, int32_t* sel,
                             int sel_stride, int32_t* sel_count, int max_pages,
                             int waves_per_block, hipStream_t s);
hipError_t launch_attention_gqa(const Meta& m, const vx_geom& g, const void* q,
                                const void* k_pool, const void* v_pool, const int32_t* sel,
                                int sel_stride, const int32_t* sel_count, float sm_scale,
                                int num_splits, int pages_per_split, float* out, float* lse,
                                float* part_o, float* part_ml, int max_pages, hipStream_t s);
hipError_t launch_attention_mla(const Meta& m, const vx_geom& g, const void* q,
                                const void* k_pool, const int32_t* sel, int sel_stride,
                                const int32_t* sel_count, float sm_scale, int num_splits,
                                int pages_per_split, float* out, float* lse, float* part_o,
                                float* part_ml, hipStream_t s);
// MLA step after scoring in one kernel: every split block selects its
// sequence's pages from the scores (block s == 0 writes sel / sel_count),
// then attends over its share. Fusable when the keys and the selection fit
// the kernel's LDS.
bool decode_step_mla_fusable(int max_pages, int sel_stride);
hipError_t launch_decode_step_mla(const Meta& m, const vx_geom& g, const void* q,
                                  const void* k_pool, const float* scores, int k, int n_sink,
                                  int n_local, int mode, const uint32_t* rnd, int32_t* sel,
                                  int sel_stride, int32_t* sel_count, float sm_scale,
                                  int num_splits, float* out, float* lse, float* part_o,
                                  float* part_ml, int max_pages, int refresh, float* cent32,
                                  uint16_t* cent_bf16, float score_scale, hipStream_t s);
// Quest-style page bounds (GQA): rebuild every entry (first_token NULL) or
// refresh each sequence's pages from first_token[b]; bounds in the KV dtype.
hipError_t launch_bounds_update(const Meta& m, const vx_geom& g, const void* k_pool,
                                const int32_t* first_token, void* bounds, hipStream_t s);
// Upper-bound page scores from the bounds; refresh != 0 first recomputes each
// sequence's newest page's bounds from k_pool.
hipError_t launch_bound_scores(const Meta& m, const vx_geom& g, const void* q, const void* k_pool,
                               void* bounds, int refresh, float scale, float* scores,
                               int max_pages, hipStream_t s);
hipError_t launch_merge(int batch, int hq, int dv, int num_splits, const float* part_o,
                        const float* part_ml, float* out, float* lse, hipStream_t s);

// Largest selection one attention split streams: its page list sits in LDS,
// one entry per thread of the block that fills it (blocks have >= 256).
constexpr int kMaxPagesPerSplit = 256;
// Waves per block of the GQA bf16 attention (standalone and whole-step
// kernels alike, so both sum in the same order): 16 for short segments with
// G <= 4 (more chunks in flight at once), else 8.
constexpr int kMaxSegPagesFor16 = 512;
inline int gqa_attn_waves(int G, int max_pages) {
  return (G <= 4 && max_pages <= kMaxSegPagesFor16) ? 16 : 8;
}
// Largest page capacity for which the whole-step kernel keeps every entry's
// key and physical page in LDS.
constexpr int kMaxFusedStepPages = 4096;
// Largest batch the whole-step kernel ranks itself (each block compares every
// sequence's page count against every other's).
constexpr int kMaxPairedBatch = 256;
// LDS words a segment's selection needs besides its keys: three 256-word
// digit histograms and the block select's 2 * 16 reduction words.
constexpr int kSelectHistWords = 3 * 256;  // three rotating digit histograms
constexpr int kSelectExtraWords = kSelectHistWords + 32;
// Segments longer than this are selected by every wave of the block.
constexpr int kBlockSelectMin = 256;
// Largest per-sequence page count the top-k supports (LDS resident keys).
constexpr int kMaxTopkPages = 16000;
// Largest batch whose sequences the planner orders longest first.
constexpr int kMaxOrderedBatch = 1024;


}  // namespace vx
