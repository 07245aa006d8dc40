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
// dealt to the block's NW waves in the ChunkDeal order below; the waves'
// (m, l, o) merge in LDS at the end.
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

// Element e of a and of b (16-bit elements) as the low and high half of one
// word: one byte permute.
VX_DEV uint32_t pair16(const u32x4& a, const u32x4& b, int e) {
  const int k = e >> 1;
  const uint32_t wa = k == 0 ? a.x : k == 1 ? a.y : k == 2 ? a.z : a.w;
  const uint32_t wb = k == 0 ? b.x : k == 1 ? b.y : k == 2 ? b.z : b.w;
  return __builtin_amdgcn_perm(wb, wa, (e & 1) ? 0x07060302u : 0x05040100u);
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

// Order in which a block's NW waves take the chunks of a page list of np
// pages (CPP chunks each): the chunks of the first and last page (the sink
// and the newest page when those are forced, so known before any selection)
// go to the waves from the top, wave NW-1 first, and each such wave takes
// them before its other chunks; the chunks in between are dealt round-robin
// from wave 0. Every caller of a given list uses this order, so the waves
// accumulate the same chunks in the same order.
template <int CPP>
struct ChunkDeal {
  int np, nf, nm;  // pages, first/last-page chunks, chunks in between
  VX_DEV ChunkDeal(int np_) : np(np_), nf((np_ >= 2 ? 2 : np_) * CPP), nm(np_ * CPP - nf) {}
  // chunk index of end chunk f (< nf): pages 0 then np - 1
  VX_DEV int end_chunk(int f) const { return f < CPP ? f : (np - 1) * CPP + (f - CPP); }
};

// Per-wave online-softmax state of mfma_attend.
struct MfmaState {
  f32x4_t o[8];
  float mrow[4], lrow[4];
  VX_DEV void init() {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) { mrow[i] = kNegBig; lrow[i] = 0.f; }
  }
};

// One 16-token chunk (tokens `first` .. first+15 of physical page `phys`,
// nvc of them valid) of KV head g: load, then q.k^T, online softmax and P.V
// into st. One chunk in flight per wave: its loads are issued, then it is
// consumed, so no load register lives across chunks.
template <int G, int P, int NW>
VX_DEV void mfma_chunk(MfmaShared<G, NW>& sm, MfmaState& st, int phys, int first, int nvc, int g,
                       int hkv, const u32x4* qa, const uint16_t* __restrict__ kp,
                       const uint16_t* __restrict__ vp, float qscale) {
  constexpr int DK = 128;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  uint16_t* pw = sm.ptile[w];
  const size_t base = ((size_t)phys * hkv + g) * ((size_t)P * DK) + (size_t)first * DK;
  u32x4 kr[DK / 32], vr[4];
  {
    const uint16_t* kc = kp + base + (size_t)col * DK + 8 * q4;
    const uint16_t* vc = vp + base + (size_t)(4 * q4) * DK + 8 * col;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) kr[ks] = __builtin_nontemporal_load((const u32x4*)(kc + 32 * ks));
#pragma unroll
    for (int r = 0; r < 4; ++r) vr[r] = __builtin_nontemporal_load((const u32x4*)(vc + r * DK));
  }
  f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[ks]),
                                                   __builtin_bit_cast(bf16x8_t, kr[ks]), sacc,
                                                   0, 0, 0);
  // Rows 4 q4 + i of the tile; with G < 4 only i < G of the lanes with
  // q4 == 0 are heads, so the softmax runs for those rows only. The other
  // rows' P entries are never written, which only touches output rows past
  // G (an MFMA output row depends on its own A row alone), never read.
  constexpr int NI = G < 4 ? G : 4;
  const bool tok_ok = col < nvc;
  float alpha[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float z = tok_ok ? sacc[i] * qscale : -INFINITY;
    const float mnew = fmaxf(st.mrow[i], group_max<16>(z));
    alpha[i] = __builtin_amdgcn_exp2f(st.mrow[i] - mnew);
    grow = grow || (mnew > st.mrow[i]);
    const float pv = __builtin_amdgcn_exp2f(z - mnew);  // in [0, 1], never NaN
    st.lrow[i] = fmaf(st.lrow[i], alpha[i], group_sum<16>(pv));
    st.mrow[i] = mnew;
    // round to nearest even (v_cvt_pk_bf16_f32)
    pw[(4 * q4 + i) * kPRow + col] = __builtin_bit_cast(uint16_t, (__bf16)pv);
  }
  if (__ballot(grow)) {  // rescale only when some row's maximum moved
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < NI; ++i) st.o[e][i] *= alpha[i];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint2 pa = *(const uint2*)(pw + col * kPRow + 4 * q4);
  u32x4 v[4];
  if (nvc >= 16) {  // a whole chunk (uniform): no value row to clear
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = vr[r];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (4 * q4 + r < nvc) ? vr[r] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t b01 = pair16(v[0], v[1], e);
    const uint32_t b23 = pair16(v[2], v[3], e);
    st.o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(bf16x4_t, pa), __builtin_bit_cast(bf16x4_t, uint2{b01, b23}), st.o[e],
        0, 0, 0);
  }
  __builtin_amdgcn_wave_barrier();  // P tile reads done before the next chunk writes it
}

// This wave's end chunks of the deal (chunks of the first and last page of
// the list, given as physical page and valid tokens of each).
template <int G, int P, int NW>
VX_DEV void mfma_end_chunks(MfmaShared<G, NW>& sm, MfmaState& st, const ChunkDeal<P / 16>& d,
                            int phys0, int nv0, int phys1, int nv1, int g, int hkv,
                            const u32x4* qa, const uint16_t* __restrict__ kp,
                            const uint16_t* __restrict__ vp, float qscale) {
  constexpr int CPP = P / 16;
  const int w = threadIdx.x >> 6;
  for (int f = NW - 1 - w; f < d.nf; f += NW) {
    const bool first = f < CPP;
    const int cp = first ? f : f - CPP;
    mfma_chunk<G, P, NW>(sm, st, first ? phys0 : phys1, 16 * cp, (first ? nv0 : nv1) - 16 * cp, g,
                         hkv, qa, kp, vp, qscale);
  }
}

// This wave's chunks in between (pages 1 .. np-2 of the list).
template <int G, int P, int NW>
VX_DEV void mfma_mid_chunks(MfmaShared<G, NW>& sm, MfmaState& st, const ChunkDeal<P / 16>& d,
                            const int* pg_phys, const int* pg_nv, int g, int hkv,
                            const u32x4* qa, const uint16_t* __restrict__ kp,
                            const uint16_t* __restrict__ vp, float qscale) {
  constexpr int CPP = P / 16;
  const int w = threadIdx.x >> 6;
  for (int m = w; m < d.nm; m += NW) {
    const int c = CPP + m;
    const int pg = c / CPP, cp = c % CPP;
    mfma_chunk<G, P, NW>(sm, st, pg_phys[pg], 16 * cp, pg_nv[pg] - 16 * cp, g, hkv, qa, kp, vp,
                         qscale);
  }
}

// The waves' states merged in LDS; S == 1 writes out / lse (lse nullable),
// otherwise split s's unnormalised (o, m, l) to part_o / part_ml. Called by
// every thread of the block.
template <int G, int NW>
VX_DEV void mfma_finish(MfmaShared<G, NW>& sm, const MfmaState& st, int b, int g, int hkv, int S,
                        int s, float* __restrict__ out, float* __restrict__ lse,
                        float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int DK = 128;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  const int hq = hkv * G;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    if (h < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.red_o[w][h][8 * col + e] = st.o[e][i];
      if (col == 0) {
        sm.red_ml[w][h][0] = st.mrow[i];
        sm.red_ml[w][h][1] = st.lrow[i];
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
      __builtin_nontemporal_store(acc, part_o + ps * DK + d);  // read once, by the merge
      if (d == 0) {
        part_ml[2 * ps] = mmax;
        part_ml[2 * ps + 1] = lsum;
      }
    }
  }
}

// Attention of query heads g*G .. g*G+G-1 of sequence b over the np pages
// pg_phys[0..np) (physical ids, pg_nv valid tokens each), listed in LDS and
// visible to the whole block, in the ChunkDeal order. S == 1: writes out /
// lse (lse nullable); otherwise split s's unnormalised (o, m, l) to part_o /
// part_ml.
template <int G, int P, int NW>
VX_DEV void mfma_attend(MfmaShared<G, NW>& sm, const int* pg_phys, const int* pg_nv, int np, int b,
                        int g, int hkv, const u32x4* qa, const uint16_t* __restrict__ kp,
                        const uint16_t* __restrict__ vp, float qscale, int S, int s,
                        float* __restrict__ out, float* __restrict__ lse,
                        float* __restrict__ part_o, float* __restrict__ part_ml) {
  static_assert(G >= 1 && G <= 16, "group");
  MfmaState st;
  st.init();
  const ChunkDeal<P / 16> d(np);
  if (np > 0)
    mfma_end_chunks<G, P, NW>(sm, st, d, pg_phys[0], pg_nv[0], pg_phys[np - 1], pg_nv[np - 1], g,
                              hkv, qa, kp, vp, qscale);
  mfma_mid_chunks<G, P, NW>(sm, st, d, pg_phys, pg_nv, g, hkv, qa, kp, vp, qscale);
  mfma_finish<G, NW>(sm, st, b, g, hkv, S, s, out, lse, part_o, part_ml);
}

}  // namespace vx
