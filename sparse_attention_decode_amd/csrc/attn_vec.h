// Vector-ALU attention over a list of pages for one (sequence, KV head),
// used by the stand-alone GQA attention kernel (fp32 keys or Dk = 64) and by
// the whole-step kernel for those geometries, so both sum in the same order.
//
// A block of kVecWaves waves walks the pages as 16-token chunks dealt
// round-robin to the waves; each wave loads a batch of chunks, then consumes
// it. A chunk is read with 16-byte loads, lane l covering bytes
// [16 l, 16 l + 16) of every 1 KB, so each load instruction is 1 KB
// contiguous. That puts each token row across LPR = Dk / E lanes (E elements
// per 16 B) and TPI = 64 / LPR tokens in one instruction. q.k is a per-lane
// partial (v_dot2_f32_bf16 for bf16) reduced over the LPR lanes with DPP;
// each group of LPR lanes ("row") keeps its own online-softmax state
// (m, l, o) for the tokens it holds, so V needs no cross-lane traffic. Rows
// merge inside the wave, waves merge in LDS; the block writes the output (one
// split) or its split's partial. Logits are in log2 units.
#pragma once

#include "vx_internal.h"

namespace vx {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename KV> struct KVTraits;
template <> struct KVTraits<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void to_f32(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};
template <> struct KVTraits<uint16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void to_f32(const u32x4& w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
};

constexpr int kVecWaves = 8;  // waves per vector attention block
constexpr int kVecBatch = 1;  // chunks in flight per wave (short rows)

template <typename QT, typename KV, int G>
struct VecQuery {
  float qf[G][KVTraits<KV>::E];          // fp32 path: query times the scale
  uint32_t qp[G][KVTraits<KV>::E / 2];   // bf16 v_dot2 path: packed pairs
};

template <int G, int DK>
struct VecShared {
  float red_o[kVecWaves][G][DK];
  float red_ml[kVecWaves][G][2];
};

// This lane's share of the group's query rows.
template <typename QT, typename KV, int G, int DK>
VX_DEV void vec_load_q(const QT* __restrict__ q, int b, int g, int hkv, float qscale,
                       VecQuery<QT, KV, G>& vq) {
  constexpr int E = KVTraits<KV>::E;
  constexpr int LPR = DK / E;
  constexpr bool kDot2 = sizeof(KV) == 2 && sizeof(QT) == 2;
  const int lane = threadIdx.x & 63;
  const int hq = hkv * G;
  const int dofs = (lane % LPR) * E;
  // Query rows of the group (log2 units): packed bf16 pairs for v_dot2, or fp32.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const QT* qh = q + ((size_t)b * hq + g * G + h) * DK + dofs;
    if constexpr (kDot2) {
#pragma unroll
      for (int e = 0; e < E / 2; ++e) vq.qp[h][e] = ((const uint32_t*)qh)[e];
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (sizeof(QT) == 2) vq.qf[h][e] = bf16_to_f32(qh[e]) * qscale;
        else vq.qf[h][e] = (float)qh[e] * qscale;
      }
    }
  }
}

// Attention of query heads g*G .. g*G+G-1 of sequence b over the np pages
// (physical page, valid tokens) listed in LDS; S == 1 writes out / lse, else
// split s's partial (o, m, l). The caller makes the page list visible first.
template <typename QT, typename KV, int G, int DK, int P>
VX_DEV void vec_attend(VecShared<G, DK>& sm, const int* pg_phys, const int* pg_nv, int np, int b,
                       int g, int hkv, const VecQuery<QT, KV, G>& vq, const KV* __restrict__ kp,
                       const KV* __restrict__ vp, float qscale, int S, int s,
                       float* __restrict__ out, float* __restrict__ lse,
                       float* __restrict__ part_o, float* __restrict__ part_ml) {
  using T = KVTraits<KV>;
  constexpr int E = T::E;
  constexpr int LPR = DK / E;      // lanes per token row
  constexpr int TPI = 64 / LPR;    // tokens per load instruction
  constexpr int CT = 16;           // tokens per chunk
  constexpr int CH = CT / TPI;     // load instructions per chunk (per K and per V)
  constexpr int CPP = P / CT;      // chunks per page
  constexpr bool kDot2 = sizeof(KV) == 2 && sizeof(QT) == 2;
  static_assert(64 % LPR == 0 && CT % TPI == 0 && P % CT == 0, "layout");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hq = hkv * G;
  const int row = lane / LPR;
  const int dofs = (lane % LPR) * E;
  const auto& qf = vq.qf;
  const auto& qp = vq.qp;
  (void)qf;
  (void)qp;

  float mrow[G], lrow[G], o[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mrow[h] = kNegBig;
    lrow[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[h][e] = 0.f;
  }

  const int nchunks = np * CPP;
  const size_t head_stride = (size_t)P * DK;
  auto chunk_nv = [&](int c) { return pg_nv[c / CPP] - (c % CPP) * CT; };
  auto load_chunk = [&](int c, u32x4* kr, u32x4* vr) {
    const size_t base = ((size_t)pg_phys[c / CPP] * hkv + g) * head_stride + (size_t)(c % CPP) * CT * DK;
    const u32x4* kc = (const u32x4*)(kp + base);
    const u32x4* vc = (const u32x4*)(vp + base);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      kr[i] = __builtin_nontemporal_load(kc + i * 64 + lane);
      vr[i] = __builtin_nontemporal_load(vc + i * 64 + lane);
    }
  };
  // No early exit: an empty chunk is consumed fully masked, so every slot's
  // loads are waited on in one place and the prefetch ring stays pipelined.
  auto consume = [&](int c, const u32x4* kr, const u32x4* vr) {
    const int nvc = chunk_nv(c);
    const bool full = nvc >= CT;
    float z[CH][G];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool valid = full || (i * TPI + row) < nvc;
      if constexpr (kDot2) {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[h][e]),
                                                  __builtin_bit_cast(bf16x2_t, kw[e]), acc, false);
          acc = group_sum<LPR>(acc) * qscale;
          z[i][h] = valid ? acc : -INFINITY;
        }
      } else {
        float kf[E];
        T::to_f32(kr[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) acc = fmaf(qf[h][e], kf[e], acc);
          acc = group_sum<LPR>(acc);
          z[i][h] = valid ? acc : -INFINITY;
        }
      }
    }
    float pr[CH][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = z[0][h];
#pragma unroll
      for (int i = 1; i < CH; ++i) mx = fmaxf(mx, z[i][h]);
      const float mnew = fmaxf(mrow[h], mx);
      const float alpha = __builtin_amdgcn_exp2f(mrow[h] - mnew);
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        pr[i][h] = __builtin_amdgcn_exp2f(z[i][h] - mnew);
        lsum += pr[i][h];
      }
      lrow[h] = fmaf(lrow[h], alpha, lsum);
      mrow[h] = mnew;
#pragma unroll
      for (int e = 0; e < E; ++e) o[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      float vf[E];
      T::to_f32(vr[i], vf);
      if (!full && (i * TPI + row) >= nvc) {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = fmaf(pr[i][h], vf[e], o[h][e]);
    }
  };

  // Batches of NB chunks (see attn_gqa_mfma_kernel): loads first, then use.
  constexpr int NB = CH >= 8 ? 1 : kVecBatch;
  const int my_n = nchunks > w ? (nchunks - w + kVecWaves - 1) / kVecWaves : 0;
  for (int j0 = 0; j0 < my_n; j0 += NB) {
    u32x4 kr[NB][CH], vr[NB][CH];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      load_chunk(w + min(j0 + u, my_n - 1) * kVecWaves, kr[u], vr[u]);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (j0 + u < my_n) consume(w + (j0 + u) * kVecWaves, kr[u], vr[u]);
  }

  // Merge the TPI rows of each head inside the wave (lanes l ^ LPR, ...).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) {
      const float mo = __shfl_xor(mrow[h], x);
      const float lo = __shfl_xor(lrow[h], x);
      const float mnew = fmaxf(mrow[h], mo);
      const float a = __builtin_amdgcn_exp2f(mrow[h] - mnew);
      const float bsc = __builtin_amdgcn_exp2f(mo - mnew);
      lrow[h] = lrow[h] * a + lo * bsc;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float oo = __shfl_xor(o[h][e], x);
        o[h][e] = o[h][e] * a + oo * bsc;
      }
      mrow[h] = mnew;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm.red_o[w][h][dofs + e] = o[h][e];
      if (lane == 0) {
        sm.red_ml[w][h][0] = mrow[h];
        sm.red_ml[w][h][1] = lrow[h];
      }
    }
  }
  __syncthreads();

  // Merge the waves: thread -> (head, 4 dims).
  for (int t = threadIdx.x; t < G * DK / 4; t += blockDim.x) {
    const int h = t / (DK / 4), d = (t % (DK / 4)) * 4;
    float mmax = kNegBig;
#pragma unroll
    for (int v = 0; v < kVecWaves; ++v) mmax = fmaxf(mmax, sm.red_ml[v][h][0]);
    float lsum = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < kVecWaves; ++v) {
      const float wt = __builtin_amdgcn_exp2f(sm.red_ml[v][h][0] - mmax);
      lsum = fmaf(sm.red_ml[v][h][1], wt, lsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(sm.red_o[v][h][d + e], wt, acc[e]);
    }
    const int head = g * G + h;
    if (S == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float4* dst = (float4*)(out + ((size_t)b * hq + head) * DK + d);
      *dst = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      if (lse && d == 0)
        lse[(size_t)b * hq + head] = lsum > 0.f ? (mmax + log2f(lsum)) * kLn2 : -INFINITY;
    } else {
      const size_t ps = ((size_t)b * hq + head) * S + s;
      typedef float f4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(f4v{acc[0], acc[1], acc[2], acc[3]},
                                  (f4v*)(part_o + ps * DK + d));  // read once, by the merge
      if (d == 0) {
        part_ml[2 * ps] = mmax;
        part_ml[2 * ps + 1] = lsum;
      }
    }
  }
}

}  // namespace vx
