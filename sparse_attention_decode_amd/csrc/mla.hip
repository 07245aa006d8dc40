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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ scoring
// grid (ceil(max_pages / 64), B), 4 waves; wave w scores the 16 pages
// [64 * blockIdx.x + 16 w, +16) of sequence blockIdx.y. With `refresh`, the
// block holding a sequence's newest page first recomputes that page's
// centroid (fp32 and its bf16 copy) from its keys, in token order with one
// IEEE divide per column, the cache stage's arithmetic; the barrier before
// scoring orders it before the page's bf16 row is read.
template <int MT, int KS>
__global__ __launch_bounds__(256) void scores_mla_kernel(Meta m, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ kp,
                                                         float* __restrict__ cent32,
                                                         uint16_t* __restrict__ cent, int refresh,
                                                         float scale, float* __restrict__ scores) {
  constexpr int kQPer = (16 * MT * (DK / 8) + 255) / 256;  // query vectors per thread
  __shared__ __attribute__((aligned(16))) uint16_t qs[16 * MT * ROW];
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  int n = (L + m.page_size - 1) / m.page_size;
  n = n > cap ? cap : n;
  const int blk0 = blockIdx.x * 64;
  if (blk0 >= n) return;  // whole block: no barrier reached

  // This sequence's query rows (16 * MT heads x 576): all loads issued, then stored in LDS.
  const uint16_t* qb = q + (size_t)b * (16 * MT) * DK;
  u32x4 qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int c = t + 256 * u;
    if (c < 16 * MT * (DK / 8)) qv[u] = *(const u32x4*)(qb + (c / (DK / 8)) * DK + 8 * (c % (DK / 8)));
  }
  if (refresh && n - 1 < blk0 + 64) {  // the newest page is in this block's range
    const int P = m.page_size;
    const int pn = n - 1;
    const int nv = min(P, L - pn * P);
    const int pid = phys_page(m, row0 + pn);
    const uint16_t* kb = kp + (size_t)pid * P * DK;
    for (int pr = t; pr < DK / 2; pr += 256) {
      float s0 = 0.f, s1 = 0.f;
      for (int t0 = 0; t0 < nv; t0 += 32) {
        uint32_t x[32];
#pragma unroll
        for (int u = 0; u < 32; ++u)
          if (t0 + u < nv) x[u] = *(const uint32_t*)(kb + (size_t)(t0 + u) * DK + 2 * pr);
#pragma unroll
        for (int u = 0; u < 32; ++u)
          if (t0 + u < nv) { s0 += bf16_lo(x[u]); s1 += bf16_hi(x[u]); }
      }
      const float c0 = s0 / (float)nv, c1 = s1 / (float)nv;
      const size_t o = (size_t)pid * DK + 2 * pr;
      *(float2*)(cent32 + o) = make_float2(c0, c1);
      *(uint32_t*)(cent + o) = (uint32_t)f32_to_bf16(c0) | ((uint32_t)f32_to_bf16(c1) << 16);
    }
  }
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int c = t + 256 * u;
    if (c < 16 * MT * (DK / 8)) *(u32x4*)(qs + (c / (DK / 8)) * ROW + 8 * (c % (DK / 8))) = qv[u];
  }
  __syncthreads();

  const int base = blk0 + 16 * w;
  if (base >= n) return;
  const int col = lane & 15, q4 = lane >> 4;
  const int p = base + col;
  const bool valid = p < n;
  const uint16_t* crow = cent + (size_t)(valid ? phys_page(m, row0 + p) : 0) * DK + 8 * q4;

  u32x4 bf[KS];  // KS k steps of 32 columns: 18 = all 576, 16 = the 512 latent ones
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bf[ks] = valid ? *(const u32x4*)(crow + 32 * ks) : u32x4{0u, 0u, 0u, 0u};

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* arow = qs + (16 * mt + col) * ROW + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma(*(const u32x4*)(arow + 32 * ks), bf[ks], acc[mt]);
  }
  float s = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) s += (acc[mt][0] + acc[mt][1]) + (acc[mt][2] + acc[mt][3]);
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if (lane < 16 && valid) scores[row0 + p] = s * scale;
}

// ---------------------------------------------------------------- attention
// One block (8 waves) per (sequence b, split s); the split holds a balanced
// share of the selected pages. Pages are consumed as 64-token chunks. Each
// chunk is staged in LDS twice: row-major (the B operand of q.k^T reads a
// token's 8 consecutive columns) and value columns transposed (the B operand
// of P.V reads 8 consecutive tokens of one column); the transpose is done in
// registers on 8x8 bf16 blocks, so both operands are single 16-byte LDS
// reads; in the transposed copy, the 8-token groups of column r sit at
// group index ^ ((r / 8) % 8), which spreads a wave's stores over the LDS
// banks. The next kRing chunks are in flight in registers while one is
// consumed. Logits: wave w < 4 MT computes the 16x16 tile (head tile w % MT,
// token tile w / MT); row maxima and sums are exchanged through LDS. P.V:
// wave w owns head tile w % MT and value columns [part * 512 / NP, +512 / NP)
// with NP = 8 / MT, so its accumulators stay small enough for two waves per
// SIMD.
constexpr int kMlaWaves = 8;
constexpr int CHT = 64;                 // tokens per chunk
constexpr int NTT = CHT / 16;           // token tiles per chunk
#ifndef VX_MLA_RING
#define VX_MLA_RING 1
#endif
constexpr int kRing = VX_MLA_RING;      // chunks in flight per block
constexpr int VT_ROW = CHT + 8;         // padded transposed-V row (bf16), 144 B
constexpr int PROW = CHT + 8;           // padded P row (bf16)

__device__ __forceinline__ uint32_t half_of(const u32x4& v, int e) {
  const uint32_t wv = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (wv >> 16) : (wv & 0xffffu);
}

template <int MT>
__global__ __launch_bounds__(64 * kMlaWaves) void attn_mla_kernel(
    Meta m, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const int32_t* __restrict__ sel, int stride, const int32_t* __restrict__ sel_count,
    float qscale, int S, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int HQ = 16 * MT;
  constexpr int NP = kMlaWaves / MT;  // value-column parts
  constexpr int NT2 = DV / NP / 16;   // 16-column tiles per wave
  static_assert(DV / 8 * (CHT / 8) == 64 * kMlaWaves, "one 8x8 staging block per thread");
  static_assert(CHT * 8 == 64 * kMlaWaves, "one rope vector per thread");
  __shared__ __attribute__((aligned(16))) uint16_t krow[CHT * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt[DV * VT_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t pl[MT][16 * PROW];
  __shared__ float rmax[MT][NTT][16];
  __shared__ float rsum[MT][NTT][16];
  __shared__ int pg_phys[kMaxPagesPerSplit];
  __shared__ int pg_nv[kMaxPagesPerSplit];

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  const int mt = w % MT, part = w / MT;
  const bool qk_wave = w < NTT * MT;
  const int nt = w / MT;  // token tile of the logit tile (qk waves)
  const int item = blockIdx.x;
  const int s = item % S, b = item / S;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  const int count = cap > 0 ? min(sel_count[b], stride) : 0;
  const int p0 = (int)(((long)count * s) / S);
  const int np = min((int)(((long)count * (s + 1)) / S) - p0, kMaxPagesPerSplit);
  const int P = m.page_size;  // 64 (checked on the host): one chunk per page

  static_assert(kMaxPagesPerSplit <= 64 * kMlaWaves, "one page-list entry per thread");
  if (t < np) {
    int lp = sel[(size_t)b * stride + p0 + t];
    lp = lp < 0 ? 0 : (lp >= cap ? cap - 1 : lp);
    pg_phys[t] = phys_page(m, row0 + lp);
    pg_nv[t] = max(0, min(P, L - lp * P));
  }

  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = q + ((size_t)b * HQ + 16 * mt + col) * DK + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *(const u32x4*)(qrow + 32 * ks);
  }
  f32x4 o[NT2];
#pragma unroll
  for (int x = 0; x < NT2; ++x) o[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { mrow[i] = kNegBig; lrow[i] = 0.f; }
  __syncthreads();  // page list ready

  const int cpp = P / CHT;
  const int nchunks = np * cpp;
  // Valid tokens of chunk c; chunks past the end (the ring's tail) are empty
  // and contribute exactly nothing (p = 0, alpha = 1).
  auto chunk_valid = [&](int c) {
    return c < nchunks ? min(CHT, pg_nv[c / cpp] - (c % cpp) * CHT) : 0;
  };
  // staging roles: an 8x8 (token x column) block of value columns + one rope vector
  const int dg = t & 63, tg = t >> 6;      // columns 8 dg.., tokens 8 tg..
  const int rr = t >> 3, rg = t & 7;       // rope: token rr, columns 512 + 8 rg..
  // Ring of kRing chunks in flight; a load past the end re-reads the last chunk.
  u32x4 vb[kRing][8], rp[kRing];
  auto prefetch = [&](int c, u32x4* v, u32x4& r) {
    c = min(c, nchunks - 1);
    const uint16_t* src = kp + ((size_t)pg_phys[c / cpp] * P + (size_t)(c % cpp) * CHT) * DK;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = __builtin_nontemporal_load((const u32x4*)(src + (8 * tg + i) * DK + 8 * dg));
    r = __builtin_nontemporal_load((const u32x4*)(src + rr * DK + DV + 8 * rg));
  };

  const int dcol0 = part * (DV / NP);
  if (nchunks > 0) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) prefetch(d, vb[d], rp[d]);
  }
  for (int c0 = 0; c0 < nchunks; c0 += kRing) {
#pragma unroll
  for (int d = 0; d < kRing; ++d) {
    const int c = c0 + d;
    const int nv = chunk_valid(c);
    __syncthreads();  // (A) previous chunk fully consumed
    {
      u32x4 x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = (8 * tg + i < nv) ? vb[d][i] : u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)(krow + (8 * tg + i) * ROW + 8 * dg) = x[i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x4 y;
        y.x = half_of(x[0], e) | (half_of(x[1], e) << 16);
        y.y = half_of(x[2], e) | (half_of(x[3], e) << 16);
        y.z = half_of(x[4], e) | (half_of(x[5], e) << 16);
        y.w = half_of(x[6], e) | (half_of(x[7], e) << 16);
        *(u32x4*)(vt + (8 * dg + e) * VT_ROW + 8 * (tg ^ (dg & 7))) = y;
      }
      *(u32x4*)(krow + rr * ROW + DV + 8 * rg) = (rr < nv) ? rp[d] : u32x4{0u, 0u, 0u, 0u};
    }
    prefetch(c + kRing, vb[d], rp[d]);
    __syncthreads();  // (B) chunk c staged

    float z[4];
    if (qk_wave) {
      f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
      const uint16_t* kr = krow + (16 * nt + col) * ROW + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ks += 2) {
        a0 = mfma(qf[ks], *(const u32x4*)(kr + 32 * ks), a0);
        a1 = mfma(qf[ks + 1], *(const u32x4*)(kr + 32 * (ks + 1)), a1);
      }
      const bool ok = 16 * nt + col < nv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = ok ? (a0[i] + a1[i]) * qscale : -INFINITY;
        const float mx = group_max<16>(z[i]);
        if (col == 0) rmax[mt][nt][4 * q4 + i] = mx;
      }
    }
    __syncthreads();  // (C) row maxima of every token tile
    float mnew[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * q4 + i;
      float mx = rmax[mt][0][r];
#pragma unroll
      for (int u = 1; u < NTT; ++u) mx = fmaxf(mx, rmax[mt][u][r]);
      mnew[i] = fmaxf(mrow[i], mx);
      alpha[i] = __builtin_amdgcn_exp2f(mrow[i] - mnew[i]);
    }
    if (qk_wave) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(z[i] - mnew[i]);
        const float sum = group_sum<16>(e);
        if (col == 0) rsum[mt][nt][4 * q4 + i] = sum;
        pl[mt][(4 * q4 + i) * PROW + 16 * nt + col] = f32_to_bf16(e);
      }
    }
    __syncthreads();  // (D) P and row sums ready
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * q4 + i;
      float sum = rsum[mt][0][r];
#pragma unroll
      for (int u = 1; u < NTT; ++u) sum += rsum[mt][u][r];
      lrow[i] = lrow[i] * alpha[i] + sum;
      mrow[i] = mnew[i];
    }
#pragma unroll
    for (int x = 0; x < NT2; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[x][i] *= alpha[i];
#pragma unroll
    for (int k2 = 0; k2 < CHT / 32; ++k2) {
      const u32x4 pa = *(const u32x4*)(pl[mt] + col * PROW + 32 * k2 + 8 * q4);
#pragma unroll
      for (int x = 0; x < NT2; ++x)
      {
        const int r = dcol0 + 16 * x + col;  // value column; its token groups are swizzled
        o[x] = mfma(pa, *(const u32x4*)(vt + r * VT_ROW + 8 * ((4 * k2 + q4) ^ ((r >> 3) & 7))),
                    o[x]);
      }
    }
  }
  }

  // results: rows 4*q4 + i of head tile mt, columns dcol0 + 16 x + col
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 16 * mt + 4 * q4 + i;
    if (S == 1) {
      const float inv = lrow[i] > 0.f ? 1.f / lrow[i] : 0.f;
      float* dst = out + ((size_t)b * HQ + head) * DV + dcol0 + col;
#pragma unroll
      for (int x = 0; x < NT2; ++x) dst[16 * x] = o[x][i] * inv;
      if (lse && part == 0 && col == 0)
        lse[(size_t)b * HQ + head] = lrow[i] > 0.f ? (mrow[i] + log2f(lrow[i])) * kLn2 : -INFINITY;
    } else {
      const size_t ps = ((size_t)b * HQ + head) * S + s;
      float* dst = part_o + ps * DV + dcol0 + col;
#pragma unroll
      for (int x = 0; x < NT2; ++x) dst[16 * x] = o[x][i];
      if (part == 0 && col == 0) {
        part_ml[2 * ps] = mrow[i];
        part_ml[2 * ps + 1] = lrow[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_scores_mla_sized(const Meta& m, const vx_geom& g, const void* q,
                                   const void* k_pool, float* cent32, uint16_t* cent_bf16,
                                   int refresh, float scale, float* scores, int max_pages,
                                   hipStream_t s) {
  if (m.nnz == 0 || m.batch == 0) return hipSuccess;
  dim3 grid((max_pages + 63) / 64, m.batch), block(256);
  const bool latent_only = g.score_dim == DV;
#define VX_MLA_SC(MT, KS)                                                                     \
  hipLaunchKernelGGL((scores_mla_kernel<MT, KS>), grid, block, 0, s, m, (const uint16_t*)q,  \
                     (const uint16_t*)k_pool, cent32, cent_bf16, refresh, scale, scores)
  if (g.num_q_heads == 32) {
    if (latent_only) VX_MLA_SC(2, DV / 32); else VX_MLA_SC(2, KSTEPS);
  } else if (g.num_q_heads == 16) {
    if (latent_only) VX_MLA_SC(1, DV / 32); else VX_MLA_SC(1, KSTEPS);
  } else {
    return hipErrorInvalidValue;
  }
#undef VX_MLA_SC
  return hipGetLastError();
}

hipError_t launch_attention_mla(const Meta& m, const vx_geom& g, const void* q,
                                const void* k_pool, const int32_t* sel, int sel_stride,
                                const int32_t* sel_count, float sm_scale, int num_splits,
                                int pages_per_split, float* out, float* lse, float* part_o,
                                float* part_ml, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  const float qscale = sm_scale * kLog2e;
  dim3 grid(m.batch * num_splits), block(64 * kMlaWaves);
  if (g.num_q_heads == 32)
    hipLaunchKernelGGL(attn_mla_kernel<2>, grid, block, 0, s, m, (const uint16_t*)q,
                       (const uint16_t*)k_pool, sel, sel_stride, sel_count, qscale, num_splits,
                       out, lse, part_o, part_ml);
  else if (g.num_q_heads == 16)
    hipLaunchKernelGGL(attn_mla_kernel<1>, grid, block, 0, s, m, (const uint16_t*)q,
                       (const uint16_t*)k_pool, sel, sel_stride, sel_count, qscale, num_splits,
                       out, lse, part_o, part_ml);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vx
