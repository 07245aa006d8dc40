// Exact softmax attention of one GQA group over a list of pages, bf16,
// Dk = Dv = 128, on the matrix cores (Vortex paper note, "System design >
// 1. vFlow": exact attention on the selected blocks). Shared by the split-K
// attention kernel and the whole-step kernel.
//
// The group's query heads (G <= 16, padded to 16 rows) meet each 16-token
// chunk as follows.
//   q.k^T  v_mfma_f32_16x16x32_bf16: A = query rows (lane: head l%16, dims
//          8 q4 + 32 ks..), B = key rows straight from HBM (lane: token l%16,
//          the same dims) -> S[head 4 q4 + i][token l%16].
//   P.V    v_mfma_f32_16x16x16_bf16: lane (q4, c) loads tokens 4 q4 .. 4 q4+3,
//          dims 8 c .. 8 c+7 (four 16-byte loads, whole 256-byte rows per
//          instruction). Taking N-tile e's columns as dims {8 c + e}, the B
//          fragment is element e of the lane's four rows; P reaches the A
//          layout (head l%16, tokens 4 q4..) through a 16x16 LDS tile.
//   -> O[head 4 q4 + i][dim 8 c + e] in accumulator e.
// Vector work per chunk is the online softmax only (log2 units). Chunks are
// dealt round-robin to the block's NW waves; the waves' (m, l, o) merge in
// LDS at the end.
#pragma once

#include "vx_internal.h"

namespace vx {

constexpr int kPRow = 20;  // padded row of a wave's P tile (bf16)

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// LDS of mfma_attend for NW waves.
template <int G, int NW>
struct MfmaShared {
  float red_o[NW][G][128];
  float red_ml[NW][G][2];
  __attribute__((aligned(16))) uint16_t ptile[NW][16 * kPRow];
};

VX_DEV uint32_t elem16(const u32x4& v, int e) {
  const uint32_t wv = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (wv >> 16) : (wv & 0xffffu);
}

// A operand of q.k^T: head row l%16 of the group (zero past G), dims
// 32 ks + 8 q4 .. +7.
template <int G>
VX_DEV void mfma_load_q(const uint16_t* __restrict__ q, int b, int g, int hkv, u32x4* qa) {
  constexpr int DK = 128;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, q4 = lane >> 4;
  const bool real = col < G;
  const uint16_t* qh = q + ((size_t)b * hkv * G + g * G + (real ? col : 0)) * DK + 8 * q4;
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks)
    qa[ks] = real ? *(const u32x4*)(qh + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
}

// Attention of query heads g*G .. g*G+G-1 of sequence b over the np pages
// pg_phys[0..np) (physical ids, pg_nv valid tokens each), listed in LDS and
// visible to the whole block. S == 1: writes out / lse (lse nullable);
// otherwise split s's unnormalised (o, m, l) to part_o / part_ml.
template <int G, int P, int NW>
VX_DEV void mfma_attend(MfmaShared<G, NW>& sm, const int* pg_phys, const int* pg_nv, int np, int b,
                        int g, int hkv, const u32x4* qa, const uint16_t* __restrict__ kp,
                        const uint16_t* __restrict__ vp, float qscale, int S, int s,
                        float* __restrict__ out, float* __restrict__ lse,
                        float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int DK = 128;
  constexpr int CT = 16;
  constexpr int CPP = P / CT;
  static_assert(G >= 1 && G <= 16, "group");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  const int hq = hkv * G;

  f32x4_t o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { mrow[i] = kNegBig; lrow[i] = 0.f; }
  uint16_t* pw = sm.ptile[w];

  const int nchunks = np * CPP;
  const size_t head_stride = (size_t)P * DK;
  auto chunk_nv = [&](int c) { return pg_nv[c / CPP] - (c % CPP) * CT; };
  auto load_chunk = [&](int c, u32x4* kr, u32x4* vr) {
    const size_t base = ((size_t)pg_phys[c / CPP] * hkv + g) * head_stride + (size_t)(c % CPP) * CT * DK;
    const uint16_t* kc = kp + base + (size_t)col * DK + 8 * q4;
    const uint16_t* vc = vp + base + (size_t)(4 * q4) * DK + 8 * col;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) kr[ks] = __builtin_nontemporal_load((const u32x4*)(kc + 32 * ks));
#pragma unroll
    for (int r = 0; r < 4; ++r) vr[r] = __builtin_nontemporal_load((const u32x4*)(vc + r * DK));
  };
  auto consume = [&](int c, const u32x4* kr, const u32x4* vr) {
    const int nvc = chunk_nv(c);
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[ks]),
                                                     __builtin_bit_cast(bf16x8_t, kr[ks]), sacc,
                                                     0, 0, 0);
    const bool tok_ok = col < nvc;
    float alpha[4];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = tok_ok ? sacc[i] * qscale : -INFINITY;
      const float mnew = fmaxf(mrow[i], group_max<16>(z));
      alpha[i] = __builtin_amdgcn_exp2f(mrow[i] - mnew);
      grow = grow || (mnew > mrow[i]);
      const float pv = __builtin_amdgcn_exp2f(z - mnew);
      lrow[i] = fmaf(lrow[i], alpha[i], group_sum<16>(pv));
      mrow[i] = mnew;
      pw[(4 * q4 + i) * kPRow + col] = f32_to_bf16(pv);
    }
    if (__ballot(grow)) {  // rescale only when some row's maximum moved
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[e][i] *= alpha[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint2 pa = *(const uint2*)(pw + col * kPRow + 4 * q4);
    u32x4 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (4 * q4 + r < nvc) ? vr[r] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b01 = elem16(v[0], e) | (elem16(v[1], e) << 16);
      const uint32_t b23 = elem16(v[2], e) | (elem16(v[3], e) << 16);
      o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(bf16x4_t, pa), __builtin_bit_cast(bf16x4_t, uint2{b01, b23}), o[e],
          0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();  // P tile reads done before the next chunk writes it
  };

  // One chunk in flight per wave: its loads are issued, then it is consumed.
  // No load register lives across iterations, so nothing forces the compiler
  // to copy (and wait on) in-flight registers.
  const int my_n = nchunks > w ? (nchunks - w + NW - 1) / NW : 0;
  for (int j = 0; j < my_n; ++j) {
    u32x4 kr[DK / 32], vr[4];
    load_chunk(w + j * NW, kr, vr);
    consume(w + j * NW, kr, vr);
  }

  // Per-wave results of the group's heads to LDS, then merge the waves.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    if (h < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.red_o[w][h][8 * col + e] = o[e][i];
      if (col == 0) {
        sm.red_ml[w][h][0] = mrow[i];
        sm.red_ml[w][h][1] = lrow[i];
      }
    }
  }
  __syncthreads();
  // One output element per thread (the waves' sum in wave order).
  for (int t = threadIdx.x; t < G * DK; t += blockDim.x) {
    const int h = t / DK, d = t % DK;
    float mmax = kNegBig;
#pragma unroll
    for (int v = 0; v < NW; ++v) mmax = fmaxf(mmax, sm.red_ml[v][h][0]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float wt = __builtin_amdgcn_exp2f(sm.red_ml[v][h][0] - mmax);
      lsum = fmaf(sm.red_ml[v][h][1], wt, lsum);
      acc = fmaf(sm.red_o[v][h][d], wt, acc);
    }
    const int head = g * G + h;
    if (S == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      out[((size_t)b * hq + head) * DK + d] = acc * inv;
      if (lse && d == 0)
        lse[(size_t)b * hq + head] = lsum > 0.f ? (mmax + log2f(lsum)) * kLn2 : -INFINITY;
    } else {
      const size_t ps = ((size_t)b * hq + head) * S + s;
      part_o[ps * DK + d] = acc;
      if (d == 0) {
        part_ml[2 * ps] = mmax;
        part_ml[2 * ps + 1] = lsum;
      }
    }
  }
}

}  // namespace vx
