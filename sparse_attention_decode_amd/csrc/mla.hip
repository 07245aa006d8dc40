// MLA geometry: one 576-wide latent stream (512 latent + 64 rope columns)
// shared by every query head; values are the first 512 columns of each row.
//
// Vortex paper note, "Key results > MLA": the rope part matters for routing,
// so pages are scored on all 576 columns; "System design > 3. Execution
// backend" adds an attention kernel for general MLA geometry. Both kernels
// here are dense bf16 contractions across the query heads and run on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// MFMA operand layout used throughout (lane l, 16 = l % 16, q4 = l / 16):
//   A (16 x 32):  lane holds row (l % 16), k elements 8*q4 .. 8*q4+7
//   B (32 x 16):  lane holds column (l % 16), the same k elements
//   D (16 x 16):  lane holds rows 4*q4 + i (i < 4), column (l % 16)
// A and B read the k elements from the same offsets, so the contraction is
// exact whatever order the hardware sums them in.
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int DK = 576;
constexpr int DV = 512;
constexpr int KSTEPS = DK / 32;   // 18
constexpr int ROW = DK + 8;       // padded LDS row (bf16), 1168 B: 16-B aligned
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ scoring
// grid (ceil(max_pages / 64), B), 4 waves; wave w scores the 16 pages
// [64 * blockIdx.x + 16 w, +16) of sequence blockIdx.y.
template <int MT>
__global__ __launch_bounds__(256) void scores_mla_kernel(Meta m, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ cent,
                                                         float scale, float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint16_t qs[16 * MT * ROW];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  int n = (seq_len_clamped(m, b) + m.page_size - 1) / m.page_size;
  n = n > cap ? cap : n;
  const int blk0 = blockIdx.x * 64;
  if (blk0 >= n) return;  // whole block: no barrier reached

  // Stage this sequence's query rows (16 * MT heads x 576) in LDS.
  const uint16_t* qb = q + (size_t)b * (16 * MT) * DK;
  for (int c = threadIdx.x; c < 16 * MT * (DK / 8); c += 256) {
    const int h = c / (DK / 8), k8 = c % (DK / 8);
    *(u32x4*)(qs + h * ROW + 8 * k8) = *(const u32x4*)(qb + h * DK + 8 * k8);
  }
  __syncthreads();

  const int base = blk0 + 16 * w;
  if (base >= n) return;
  const int col = lane & 15, q4 = lane >> 4;
  const int p = base + col;
  const bool valid = p < n;
  const uint16_t* crow = cent + (size_t)(valid ? phys_page(m, row0 + p) : 0) * DK + 8 * q4;

  u32x4 bf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    bf[ks] = valid ? *(const u32x4*)(crow + 32 * ks) : u32x4{0u, 0u, 0u, 0u};

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* arow = qs + (16 * mt + col) * ROW + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) acc[mt] = mfma(*(const u32x4*)(arow + 32 * ks), bf[ks], acc[mt]);
  }
  float s = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) s += (acc[mt][0] + acc[mt][1]) + (acc[mt][2] + acc[mt][3]);
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if (lane < 16 && valid) scores[row0 + p] = s * scale;
}

// ---------------------------------------------------------------- attention
// One block (4 waves) per (sequence b, split s). Pages are processed as
// 32-token chunks staged in LDS; the next chunk is prefetched into registers
// while the current one is consumed. Wave w owns query-head tile
// mt = w % MT and value columns [part * DV / NP, +DV / NP), NP = 4 / MT; it
// computes its heads' logits for the whole chunk itself, so its online
// softmax state needs no exchange with other waves.
constexpr int CHT = 32;                        // tokens per chunk
constexpr int CHUNK_VEC = CHT * DK / 8;        // 16-byte vectors per chunk (2304)
constexpr int VEC_PER_THREAD = CHUNK_VEC / 256;  // 9
constexpr int PROW = CHT + 8;                  // padded P row (bf16)

template <int MT>
__global__ __launch_bounds__(256) void attn_mla_kernel(
    Meta m, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const int32_t* __restrict__ sel, int stride, const int32_t* __restrict__ sel_count,
    float qscale, int S, int pps, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int HQ = 16 * MT;
  constexpr int NP = 4 / MT;          // value-column parts
  constexpr int NT2 = DV / NP / 16;   // 16-column tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t kc[CHT * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t pl[4][16 * PROW];
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  const int mt = w % MT, part = w / MT;
  const int item = blockIdx.x;
  const int s = item % S, b = item / S;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  const int count = cap > 0 ? min(sel_count[b], stride) : 0;
  const int p0 = s * pps;
  const int np = max(0, min(count, p0 + pps) - p0);
  const int P = m.page_size;

  if (threadIdx.x < np) {
    int lp = sel[(size_t)b * stride + p0 + threadIdx.x];
    lp = lp < 0 ? 0 : (lp >= cap ? cap - 1 : lp);
    pg_phys[threadIdx.x] = phys_page(m, row0 + lp);
    pg_nv[threadIdx.x] = max(0, min(P, L - lp * P));
  }

  // Query fragments of this wave's head tile (A operand of q.k), kept in VGPRs.
  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = q + ((size_t)b * HQ + 16 * mt + col) * DK + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *(const u32x4*)(qrow + 32 * ks);
  }
  f32x4 o[NT2];
#pragma unroll
  for (int t = 0; t < NT2; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { mrow[i] = kNegBig; lrow[i] = 0.f; }
  __syncthreads();  // page list ready

  const int cpp = P / CHT;  // chunks per page
  const int nchunks = np * cpp;
  auto chunk_valid = [&](int c) { return min(CHT, pg_nv[c / cpp] - (c % cpp) * CHT); };
  auto chunk_src = [&](int c) {
    return kp + ((size_t)pg_phys[c / cpp] * P + (size_t)(c % cpp) * CHT) * DK;
  };

  u32x4 pre[VEC_PER_THREAD];
  auto prefetch = [&](int c) {
    const u32x4* src = (const u32x4*)chunk_src(c);
#pragma unroll
    for (int r = 0; r < VEC_PER_THREAD; ++r)
      pre[r] = __builtin_nontemporal_load(src + r * 256 + threadIdx.x);
  };
  auto next_valid = [&](int c) {
    while (c < nchunks && chunk_valid(c) <= 0) ++c;
    return c;
  };

  const int dcol0 = part * (DV / NP);
  uint16_t* pw = pl[w];
  int c = next_valid(0);
  if (c < nchunks) prefetch(c);
  while (c < nchunks) {
    const int nv = chunk_valid(c);
    __syncthreads();  // previous chunk fully consumed
#pragma unroll
    for (int r = 0; r < VEC_PER_THREAD; ++r) {
      const int v = r * 256 + threadIdx.x;
      const int tok = v / (DK / 8), k8 = v % (DK / 8);
      u32x4 x = pre[r];
      if (tok >= nv) x = u32x4{0u, 0u, 0u, 0u};  // rows past the sequence end
      *(u32x4*)(kc + tok * ROW + 8 * k8) = x;
    }
    const int cn = next_valid(c + 1);
    if (cn < nchunks) prefetch(cn);
    __syncthreads();  // chunk c staged

    // logits S[16 heads][32 tokens] of this wave's head tile
    f32x4 sacc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = kc + (16 * nt + col) * ROW + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) sacc[nt] = mfma(qf[ks], *(const u32x4*)(krow + 32 * ks), sacc[nt]);
    }
    // online softmax on rows 4*q4 + i; tokens 16 nt + col
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float z0 = sacc[0][i] * qscale, z1 = sacc[1][i] * qscale;
      if (col >= nv) z0 = -INFINITY;
      if (16 + col >= nv) z1 = -INFINITY;
      const float mx = group_max<16>(fmaxf(z0, z1));
      const float mnew = fmaxf(mrow[i], mx);
      alpha[i] = __builtin_amdgcn_exp2f(mrow[i] - mnew);
      const float e0 = __builtin_amdgcn_exp2f(z0 - mnew), e1 = __builtin_amdgcn_exp2f(z1 - mnew);
      lrow[i] = lrow[i] * alpha[i] + group_sum<16>(e0 + e1);
      mrow[i] = mnew;
      pw[(4 * q4 + i) * PROW + col] = f32_to_bf16(e0);
      pw[(4 * q4 + i) * PROW + 16 + col] = f32_to_bf16(e1);
    }
#pragma unroll
    for (int t = 0; t < NT2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] *= alpha[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O += P . V over the chunk's 32 tokens
    const u32x4 pa = *(const u32x4*)(pw + col * PROW + 8 * q4);
#pragma unroll
    for (int t = 0; t < NT2; ++t) {
      const int dc = dcol0 + 16 * t + col;
      uint32_t vb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = kc[(8 * q4 + 2 * e) * ROW + dc];
        const uint32_t hi = kc[(8 * q4 + 2 * e + 1) * ROW + dc];
        vb[e] = lo | (hi << 16);
      }
      o[t] = mfma(pa, u32x4{vb[0], vb[1], vb[2], vb[3]}, o[t]);
    }
    c = cn;
  }

  // results: rows 4*q4 + i of head tile mt, columns dcol0 + 16 t + col
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 16 * mt + 4 * q4 + i;
    if (S == 1) {
      const float inv = lrow[i] > 0.f ? 1.f / lrow[i] : 0.f;
      float* dst = out + ((size_t)b * HQ + head) * DV + dcol0 + col;
#pragma unroll
      for (int t = 0; t < NT2; ++t) dst[16 * t] = o[t][i] * inv;
      if (lse && part == 0 && col == 0)
        lse[(size_t)b * HQ + head] = lrow[i] > 0.f ? (mrow[i] + log2f(lrow[i])) * kLn2 : -INFINITY;
    } else {
      const size_t ps = ((size_t)b * HQ + head) * S + s;
      float* dst = part_o + ps * DV + dcol0 + col;
#pragma unroll
      for (int t = 0; t < NT2; ++t) dst[16 * t] = o[t][i];
      if (part == 0 && col == 0) {
        part_ml[2 * ps] = mrow[i];
        part_ml[2 * ps + 1] = lrow[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_scores_mla_sized(const Meta& m, const vx_geom& g, const void* q,
                                   const uint16_t* cent_bf16, float scale, float* scores,
                                   int max_pages, hipStream_t s) {
  if (m.nnz == 0 || m.batch == 0) return hipSuccess;
  dim3 grid((max_pages + 63) / 64, m.batch), block(256);
  if (g.num_q_heads == 32)
    hipLaunchKernelGGL(scores_mla_kernel<2>, grid, block, 0, s, m, (const uint16_t*)q, cent_bf16,
                       scale, scores);
  else if (g.num_q_heads == 16)
    hipLaunchKernelGGL(scores_mla_kernel<1>, grid, block, 0, s, m, (const uint16_t*)q, cent_bf16,
                       scale, scores);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention_mla(const Meta& m, const vx_geom& g, const void* q,
                                const void* k_pool, const int32_t* sel, int sel_stride,
                                const int32_t* sel_count, float sm_scale, int num_splits,
                                int pages_per_split, float* out, float* lse, float* part_o,
                                float* part_ml, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  const float qscale = sm_scale * kLog2e;
  dim3 grid(m.batch * num_splits), block(256);
  if (g.num_q_heads == 32)
    hipLaunchKernelGGL(attn_mla_kernel<2>, grid, block, 0, s, m, (const uint16_t*)q,
                       (const uint16_t*)k_pool, sel, sel_stride, sel_count, qscale, num_splits,
                       pages_per_split, out, lse, part_o, part_ml);
  else if (g.num_q_heads == 16)
    hipLaunchKernelGGL(attn_mla_kernel<1>, grid, block, 0, s, m, (const uint16_t*)q,
                       (const uint16_t*)k_pool, sel, sel_stride, sel_count, qscale, num_splits,
                       pages_per_split, out, lse, part_o, part_ml);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vx
