// Quest-style page bounds: the storage unit, the cache-stage computation of
// one unit and a unit's share of a page's upper-bound score. Shared by the
// stand-alone kernels (bounds.hip) and the per-segment indexer (index_seg.h),
// so that both give the same bits.
//
// Quest (Tang et al., "Quest: Query-Aware Sparsity for Efficient
// Long-Context LLM Inference", ICML 2024) is the other baseline of the
// Vortex paper note ("Paper context", "Key results > User-side latency").
// Layout [pool][Hkv][Dk/4][2][4] in the KV dtype: per 4 dims, their 4 key
// minima then 4 maxima.
#pragma once

#include "vx_internal.h"

namespace vx {

// Bounds unit of 4 dims: 4 minima then 4 maxima.
template <typename T> struct Unit;
template <> struct Unit<uint16_t> {
  using raw = u32x4;  // 16 bytes
  // bounds are streamed once per step: non-temporal loads
  static VX_DEV u32x4 load(const uint16_t* p) { return __builtin_nontemporal_load((const u32x4*)p); }
  static VX_DEV void widen(const u32x4& r, float* lo, float* hi) {
    lo[0] = bf16_lo(r.x); lo[1] = bf16_hi(r.x); lo[2] = bf16_lo(r.y); lo[3] = bf16_hi(r.y);
    hi[0] = bf16_lo(r.z); hi[1] = bf16_hi(r.z); hi[2] = bf16_lo(r.w); hi[3] = bf16_hi(r.w);
  }
  // exact for bf16 values
  static VX_DEV void put(uint16_t* p, const float* lo, const float* hi) {
    uint4 r;
    r.x = (uint32_t)f32_to_bf16(lo[0]) | ((uint32_t)f32_to_bf16(lo[1]) << 16);
    r.y = (uint32_t)f32_to_bf16(lo[2]) | ((uint32_t)f32_to_bf16(lo[3]) << 16);
    r.z = (uint32_t)f32_to_bf16(hi[0]) | ((uint32_t)f32_to_bf16(hi[1]) << 16);
    r.w = (uint32_t)f32_to_bf16(hi[2]) | ((uint32_t)f32_to_bf16(hi[3]) << 16);
    *(uint4*)p = r;
  }
};
template <> struct Unit<float> {
  struct raw { u32x4 lo, hi; };  // 32 bytes
  static VX_DEV raw load(const float* p) {
    return raw{__builtin_nontemporal_load((const u32x4*)p),
               __builtin_nontemporal_load((const u32x4*)(p + 4))};
  }
  static VX_DEV void widen(const raw& r, float* lo, float* hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = __uint_as_float(r.lo[i]);
      hi[i] = __uint_as_float(r.hi[i]);
    }
  }
  static VX_DEV void put(float* p, const float* lo, const float* hi) {
    *(float4*)p = make_float4(lo[0], lo[1], lo[2], lo[3]);
    *(float4*)(p + 4) = make_float4(hi[0], hi[1], hi[2], hi[3]);
  }
};

// Bounds of unit u (KV head u / (Dk/4), dims 4 * (u % (Dk/4)) ..) of one
// page over its nv valid tokens, stored at the unit's place; nv == 0 stores
// zeros. Token loads go out 16 at a time with no branch per token: indexes
// past the last token repeat it, which leaves a minimum or maximum unchanged.
template <typename KV>
VX_DEV void unit_bounds(const KV* __restrict__ kp, KV* __restrict__ bounds, int P, int hkv, int dk,
                        int pid, int nv, int u, float* lo, float* hi) {
  constexpr int kTok = 16;
  const int g = u / (dk / 4);
  const int d = 4 * (u % (dk / 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = nv > 0 ? __builtin_inff() : 0.f;
    hi[i] = nv > 0 ? -__builtin_inff() : 0.f;
  }
  const KV* base = kp + ((size_t)pid * hkv + g) * (size_t)P * dk + d;
  for (int t0 = 0; t0 < nv; t0 += kTok) {
    typename Quad<KV>::raw x[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) x[t] = Quad<KV>::load(base + (size_t)min(t0 + t, nv - 1) * dk);
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      const float4 v = Quad<KV>::widen(x[t]);
      lo[0] = fminf(lo[0], v.x); hi[0] = fmaxf(hi[0], v.x);
      lo[1] = fminf(lo[1], v.y); hi[1] = fmaxf(hi[1], v.y);
      lo[2] = fminf(lo[2], v.z); hi[2] = fmaxf(hi[2], v.z);
      lo[3] = fminf(lo[3], v.w); hi[3] = fmaxf(hi[3], v.w);
    }
  }
  Unit<KV>::put(bounds + ((size_t)pid * hkv * (dk / 4) + u) * 8, lo, hi);
}

// One unit's share of a page's bound: its 4 dims in order.
VX_DEV float unit_bound(float4 qd, const float* lo, const float* hi) {
  float acc = fmaxf(qd.x * lo[0], qd.x * hi[0]);
  acc += fmaxf(qd.y * lo[1], qd.y * hi[1]);
  acc += fmaxf(qd.z * lo[2], qd.z * hi[2]);
  acc += fmaxf(qd.w * lo[3], qd.w * hi[3]);
  return acc;
}

}  // namespace vx
