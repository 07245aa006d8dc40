// Wave-level radix top-k over one (sequence, KV head) segment of page scores.
//
// Vortex paper note, "System design > 1. vFlow": keep the top-k blocks by
// score; "System design > 3. Execution backend": top-k is the indexer's
// bottleneck, served by a radix top-k with an approximate mode (stochastic
// early termination and remapping) when recall can be traded for time.
//
// One wave per segment. Scores become order-preserving 32-bit keys in LDS
// (forced pages get key 0 and never compete). Exact mode runs 8-bit digit
// passes, most significant first, starting at the first byte where the
// smallest and largest candidate keys differ: an LDS histogram of the digit
// among keys that still match the chosen prefix, a DPP scan across the wave
// to find the digit where the count from the top reaches the remaining need
// r, and an early exit when that bucket holds exactly r keys. The
// survivors are then compacted in index order with ballot + mbcnt prefix
// sums, which yields ascending page ids and the lower-index tie-break.
// Approximate mode maps candidate scores affinely onto 256 buckets, runs one
// pass and fills the r remaining places from the boundary bucket cyclically
// from a random offset.
#pragma once

#include "vx_internal.h"

namespace vx {
namespace topk_detail {

constexpr int kU = 8;  // segment elements per lane handled per loop trip

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Order-preserving key: larger score -> larger key; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = (s == 0.f) ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t rank_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// DPP move of a 32-bit value; a lane without a source (or outside ROW_MASK)
// reads 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp0(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, true);
}

// Inclusive prefix sum over the wave (lane l: sum over lanes <= l): shifts by
// 1, 2, 4 and 8 inside rows of 16 lanes, then each row total broadcast to the
// rows above it (row_bcast:15 into rows 1 and 3, row_bcast:31 into 2 and 3).
__device__ __forceinline__ uint32_t prefix_sum(uint32_t x) {
  x += dpp0<0x111, 0xf>(x);
  x += dpp0<0x112, 0xf>(x);
  x += dpp0<0x114, 0xf>(x);
  x += dpp0<0x118, 0xf>(x);
  x += dpp0<0x142, 0xa>(x);
  x += dpp0<0x143, 0xc>(x);
  return x;
}

// Maximum over the wave (0 is the identity), same lane pattern.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp0<0x111, 0xf>(x));
  x = max(x, dpp0<0x112, 0xf>(x));
  x = max(x, dpp0<0x114, 0xf>(x));
  x = max(x, dpp0<0x118, 0xf>(x));
  x = max(x, dpp0<0x142, 0xa>(x));
  x = max(x, dpp0<0x143, 0xc>(x));
  return __builtin_amdgcn_readlane(x, 63);
}

struct Digit {
  uint32_t d;      // chosen bucket
  uint32_t above;  // keys strictly above it (among those matching the prefix)
  uint32_t count;  // keys inside it
};

// Find the bucket where the count from the top first reaches r (1 <= r <= total).
// Lane l holds buckets 4l .. 4l+3; the count of keys in buckets >= 4l is the
// wave total minus the exclusive prefix sum.
__device__ __forceinline__ Digit find_digit(const uint32_t* hist, uint32_t r, int lane) {
  const uint4 h = *(const uint4*)(hist + 4 * lane);
  const uint32_t t = h.x + h.y + h.z + h.w;
  const uint32_t pre = prefix_sum(t);
  const uint32_t total = __builtin_amdgcn_readlane(pre, 63);
  const uint32_t s0 = total - pre + t, s1 = s0 - h.x, s2 = s1 - h.y, s3 = s2 - h.z;
  int hit = -1;
  uint32_t hab = 0, hcnt = 0;
  if (s3 >= r && s3 - h.w < r) { hit = 3; hab = s3 - h.w; hcnt = h.w; }
  else if (s2 >= r && s2 - h.z < r) { hit = 2; hab = s2 - h.z; hcnt = h.z; }
  else if (s1 >= r && s1 - h.y < r) { hit = 1; hab = s1 - h.y; hcnt = h.y; }
  else if (s0 >= r && s0 - h.x < r) { hit = 0; hab = s0 - h.x; hcnt = h.x; }
  const unsigned long long found = __ballot(hit >= 0);
  const int src = __builtin_amdgcn_readfirstlane(__ffsll((long long)found) - 1);
  Digit out;
  out.d = (uint32_t)__builtin_amdgcn_readlane(4 * lane + hit, src);
  out.above = (uint32_t)__builtin_amdgcn_readlane((int)hab, src);
  out.count = (uint32_t)__builtin_amdgcn_readlane((int)hcnt, src);
  return out;
}

// Ordered compaction (ascending page index) of the survivors: forced pages,
// candidates with (key & mask) > prefix, and r of those with (key & mask) ==
// prefix taken in index order from offset `off`, cyclic over the `members`
// of that tie group. One wave; ballot + mbcnt ranks keep the order. out /
// count_out (global) and out_lds / count_lds may each be null.
__device__ __forceinline__ void wave_compact(const uint32_t* __restrict__ keys, int n, int n_sink,
                                             int n_local, uint32_t prefix, uint32_t mask,
                                             uint32_t r, uint32_t off, uint32_t members,
                                             int32_t* __restrict__ out, int stride,
                                             int32_t* __restrict__ count_out, int lane,
                                             int32_t* __restrict__ out_lds,
                                             int32_t* __restrict__ count_lds) {
  uint32_t written = 0, tie_seen = 0;
  for (int base0 = 0; base0 < n; base0 += 64 * kU) {
    uint32_t kvs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base0 + 64 * u + lane;
      kvs[u] = i < n ? keys[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
    const int i = base0 + 64 * u + lane;
    const bool in = i < n;
    const uint32_t kv = kvs[u];
    const bool forced = in && (i < n_sink || i >= n - n_local);
    const bool cand = kv != 0u;
    const bool above = cand && (kv & mask) > prefix;
    const bool tie = cand && (kv & mask) == prefix;
    const unsigned long long tmask = __ballot(tie);
    const uint32_t trank = tie_seen + rank_below(tmask);
    tie_seen += (uint32_t)__popcll(tmask);
    bool take = forced || above;
    if (tie && members) {
      // cyclic position from off: trank, off < members, so one wrap at most
      uint32_t pos = trank + members - off;
      pos = pos >= members ? pos - members : pos;
      take = take || pos < r;
    }
    const unsigned long long smask = __ballot(take);
    if (take) {
      if (out) out[written + rank_below(smask)] = i;
      if (out_lds) out_lds[written + rank_below(smask)] = i;
    }
    written += (uint32_t)__popcll(smask);
    }
  }
  if (out)
    for (int i = (int)written + lane; i < stride; i += 64) out[i] = -1;
  if (lane == 0) {
    if (count_out) *count_out = (int32_t)written;
    if (count_lds) *count_lds = (int32_t)written;
  }
}

// Number of tie ranks g in [0, x) that are taken: (g - off) mod members < r,
// the cyclic window of length r starting at off (x <= members).
__device__ __forceinline__ uint32_t ties_taken_below(uint32_t x, uint32_t r, uint32_t off,
                                                     uint32_t members) {
  const uint32_t end = off + r;  // window [off, end), wrapping past members
  uint32_t c = x > off ? min(x, min(end, members)) - off : 0u;
  if (end > members) c += min(x, end - members);
  return c;
}

// wave_compact with all NW waves of the block: wave w takes a contiguous
// range of the keys; one barrier publishes each range's counts (taken
// forced / above keys, tie members), from which every wave derives its
// output offset and its first tie rank; the order of the output is the
// same as wave_compact's. `red` is 2 * NW words of LDS.
template <int NW>
__device__ __forceinline__ void block_compact(const uint32_t* __restrict__ keys, int n, int n_sink,
                                              int n_local, uint32_t prefix, uint32_t mask,
                                              uint32_t r, uint32_t off, uint32_t members,
                                              int32_t* __restrict__ out, int stride,
                                              int32_t* __restrict__ count_out,
                                              int32_t* __restrict__ out_lds,
                                              int32_t* __restrict__ count_lds,
                                              uint32_t* __restrict__ red) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (n + NW - 1) / NW;
  const int lo = min(n, w * per), hi = min(n, lo + per);
  auto classify = [&](int i, bool& sure, bool& tie) {
    const bool in = i < hi;
    const uint32_t kv = in ? keys[i] : 0u;
    const bool forced = in && (i < n_sink || i >= n - n_local);
    const bool cand = kv != 0u;
    sure = forced || (cand && (kv & mask) > prefix);
    tie = cand && (kv & mask) == prefix;
  };
  uint32_t n_sure = 0, n_tie = 0;
  for (int base = lo; base < hi; base += 64) {
    bool sure, tie;
    classify(base + lane, sure, tie);
    n_sure += (uint32_t)__popcll(__ballot(sure));
    n_tie += (uint32_t)__popcll(__ballot(tie));
  }
  if (lane == 0) { red[w] = n_sure; red[NW + w] = n_tie; }
  __syncthreads();
  // Lane v < NW takes range v's counts; wave scans give every range's first
  // tie rank and output offset.
  const uint32_t a_v = lane < NW ? red[lane] : 0u;
  const uint32_t c_v = lane < NW ? red[NW + lane] : 0u;
  const uint32_t ties_before = prefix_sum(c_v) - c_v;
  const uint32_t taken = members ? ties_taken_below(ties_before + c_v, r, off, members) -
                                       ties_taken_below(ties_before, r, off, members)
                                 : 0u;
  const uint32_t take_v = a_v + taken;
  const uint32_t take_incl = prefix_sum(take_v);
  const uint32_t out0 = (uint32_t)__builtin_amdgcn_readlane((int)(take_incl - take_v), w);
  const uint32_t tie0 = (uint32_t)__builtin_amdgcn_readlane((int)ties_before, w);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)take_incl, NW - 1);
  uint32_t written = out0, tie_seen = tie0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    bool sure, tie;
    classify(i, sure, tie);
    const unsigned long long tmask = __ballot(tie);
    const uint32_t trank = tie_seen + rank_below(tmask);
    tie_seen += (uint32_t)__popcll(tmask);
    bool take = sure;
    if (tie && members) {
      uint32_t pos = trank + members - off;
      pos = pos >= members ? pos - members : pos;
      take = take || pos < r;
    }
    const unsigned long long smask = __ballot(take);
    if (take) {
      if (out) out[written + rank_below(smask)] = i;
      if (out_lds) out_lds[written + rank_below(smask)] = i;
    }
    written += (uint32_t)__popcll(smask);
  }
  if (out)
    for (int i = (int)total + t; i < stride; i += 64 * NW) out[i] = -1;
  if (t == 0) {
    if (count_out) *count_out = (int32_t)total;
    if (count_lds) *count_lds = (int32_t)total;
  }
}

}  // namespace topk_detail

// Select for one segment whose n keys are already in this wave's LDS
// (keys[i] = 0 for a forced page, else score_key of its score); `hist` is
// 256 words of LDS. Writes out[0..stride) and *count_out, and, when given,
// the chosen ids to out_lds[0..count) and the count to *count_lds.
__device__ __forceinline__ void wave_select_keys(uint32_t* __restrict__ keys,
                                                 uint32_t* __restrict__ hist, int n, int k,
                                                 int n_sink, int n_local, int mode,
                                                 uint32_t rnd_word, int32_t* __restrict__ out,
                                                 int stride, int32_t* __restrict__ count_out,
                                                 int lane, int32_t* __restrict__ out_lds = nullptr,
                                                 int32_t* __restrict__ count_lds = nullptr) {
  using namespace topk_detail;
  const int nf = min(n, n_sink + n_local);  // forced: a prefix and a suffix of [0, n)
  const int nc = n - nf;
  const int kk = min(k, nc);

  // Survivors: candidates with (key & mask) > prefix, plus `r` of those with
  // (key & mask) == prefix taken in index order from offset `off` (cyclic
  // over the `members` of that tie group).
  uint32_t prefix = 0, mask = 0, r = (uint32_t)kk, off = 0, members = (uint32_t)nc;
  if (kk > 0 && kk < nc) {
    // smallest and largest candidate key (forced pages hold 0 and are skipped)
    uint32_t kmax = 0u, kminc = 0u;  // kminc: max of ~key, so min = ~kminc
    for (int base = 0; base < n; base += 64 * kU) {
      uint32_t kv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + 64 * u + lane;
        kv[u] = i < n ? keys[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (kv[u]) { kmax = max(kmax, kv[u]); kminc = max(kminc, ~kv[u]); }
    }
    kmax = wave_max(kmax);
    const uint32_t kmin = ~wave_max(kminc);
    if (mode == VX_TOPK_APPROX) {
      const float mn = key_score(kmin), mx = key_score(kmax);
      const float wdt = __fsub_rn(mx, mn);
      const bool spread = wdt > 0.f;
      const float inv = spread ? __fdiv_rn(256.f, wdt) : 0.f;
      *(uint4*)(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
      wave_sync();
      for (int base = 0; base < n; base += 64 * kU) {
        uint32_t kv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = base + 64 * u + lane;
          kv[u] = i < n ? keys[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = base + 64 * u + lane;
          if (kv[u]) {
            uint32_t bk = 0;
            if (spread) {
              const float t = floorf(__fmul_rn(__fsub_rn(key_score(kv[u]), mn), inv));
              bk = t >= 255.f ? 255u : (uint32_t)t;
            }
            keys[i] = (bk << 24) | 1u;  // nonzero; digit 3 is the bucket
            atomicAdd(&hist[bk], 1u);
          }
        }
      }
      wave_sync();
      const Digit dg = find_digit(hist, r, lane);
      prefix = dg.d << 24;
      mask = 0xff000000u;
      r -= dg.above;
      members = dg.count;
      off = members ? rnd_word % members : 0u;
    } else if (kmin == kmax) {
      prefix = kmin;  // every candidate ties: index order decides
      mask = 0xffffffffu;
    } else {
      // Bytes every candidate shares need no pass: start at the first byte
      // where the smallest and largest keys differ.
      const int top = __clz(kmin ^ kmax) / 8;
      mask = top ? 0xffffffffu << (32 - 8 * top) : 0u;
      prefix = kmin & mask;
      for (int shift = 24 - 8 * top; shift >= 0; shift -= 8) {
        *(uint4*)(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        wave_sync();
        for (int base = 0; base < n; base += 64 * kU) {
          uint32_t kv[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int i = base + 64 * u + lane;
            kv[u] = i < n ? keys[i] : 0u;
          }
#pragma unroll
          for (int u = 0; u < kU; ++u)
            if (kv[u] && (kv[u] & mask) == prefix) atomicAdd(&hist[(kv[u] >> shift) & 255u], 1u);
        }
        wave_sync();
        const Digit dg = find_digit(hist, r, lane);
        prefix |= dg.d << shift;
        mask |= 255u << shift;
        r -= dg.above;
        members = dg.count;
        wave_sync();
        if (dg.count == r) break;  // the whole bucket is needed: exact already
      }
    }
  }

  topk_detail::wave_compact(keys, n, n_sink, n_local, prefix, mask, r, off, members, out, stride,
                            count_out, lane, out_lds, count_lds);
}

// Select for one segment with all NW waves of a block (every thread calls
// it; n is the same for all). keys as for wave_select_keys; `hist` is
// kSelectHistWords words of LDS, `red` 2 * NW more. The min / max sweep and each digit pass's histogram
// are shared by the waves; every wave reads the finished histogram and finds
// the same digit, so no broadcast is needed; the waves compact together.
// Same result as wave_select_keys: the selection rule has one answer.
template <int NW>
__device__ __forceinline__ void block_select_keys(uint32_t* __restrict__ keys,
                                                  uint32_t* __restrict__ hist,
                                                  uint32_t* __restrict__ red, int n, int k,
                                                  int n_sink, int n_local, int mode,
                                                  uint32_t rnd_word, int32_t* __restrict__ out,
                                                  int stride, int32_t* __restrict__ count_out,
                                                  int32_t* __restrict__ out_lds = nullptr,
                                                  int32_t* __restrict__ count_lds = nullptr) {
  using namespace topk_detail;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nf = min(n, n_sink + n_local);
  const int nc = n - nf;
  const int kk = min(k, nc);
  uint32_t prefix = 0, mask = 0, r = (uint32_t)kk, off = 0, members = (uint32_t)nc;
  if (kk > 0 && kk < nc) {
    uint32_t kmax = 0u, kminc = 0u;
    for (int i = t; i < n; i += 64 * NW) {
      const uint32_t kv = keys[i];
      if (kv) { kmax = max(kmax, kv); kminc = max(kminc, ~kv); }
    }
    kmax = wave_max(kmax);
    kminc = wave_max(kminc);
    if (lane == 0) { red[w] = kmax; red[NW + w] = kminc; }
    // histograms 0 and 1 start at zero; pass j zeroes histogram (j + 2) % 3
    if (t < 128) *(uint4*)(hist + 4 * t) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    kmax = wave_max(lane < NW ? red[lane] : 0u);
    kminc = wave_max(lane < NW ? red[NW + lane] : 0u);
    const uint32_t kmin = ~kminc;
    if (mode == VX_TOPK_APPROX) {
      const float mn = key_score(kmin), mx = key_score(kmax);
      const float wdt = __fsub_rn(mx, mn);
      const bool spread = wdt > 0.f;
      const float inv = spread ? __fdiv_rn(256.f, wdt) : 0.f;
      for (int i = t; i < n; i += 64 * NW) {
        const uint32_t kv = keys[i];
        if (kv) {
          uint32_t bk = 0;
          if (spread) {
            const float x = floorf(__fmul_rn(__fsub_rn(key_score(kv), mn), inv));
            bk = x >= 255.f ? 255u : (uint32_t)x;
          }
          keys[i] = (bk << 24) | 1u;  // nonzero; digit 3 is the bucket
          atomicAdd(&hist[bk], 1u);
        }
      }
      __syncthreads();
      const Digit dg = find_digit(hist, r, lane);
      prefix = dg.d << 24;
      mask = 0xff000000u;
      r -= dg.above;
      members = dg.count;
      off = members ? rnd_word % members : 0u;
    } else if (kmin == kmax) {
      prefix = kmin;  // every candidate ties: index order decides
      mask = 0xffffffffu;
    } else {
      const int top = __clz(kmin ^ kmax) / 8;
      mask = top ? 0xffffffffu << (32 - 8 * top) : 0u;
      prefix = kmin & mask;
      // One barrier per pass: pass j counts into histogram j % 3, which was
      // zeroed during pass j - 2 (or at the start), and zeroes histogram
      // (j + 2) % 3, whose last readers finished before this pass's barrier.
      int j = 0;
      for (int shift = 24 - 8 * top; shift >= 0; shift -= 8, ++j) {
        uint32_t* h = hist + 256 * (j % 3);
        for (int i = t; i < n; i += 64 * NW) {
          const uint32_t kv = keys[i];
          if (kv && (kv & mask) == prefix) atomicAdd(&h[(kv >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (t < 64) *(uint4*)(hist + 256 * ((j + 2) % 3) + 4 * t) = make_uint4(0u, 0u, 0u, 0u);
        const Digit dg = find_digit(h, r, lane);
        prefix |= dg.d << shift;
        mask |= 255u << shift;
        r -= dg.above;
        members = dg.count;
        if (dg.count == r) break;  // same decision in every wave
      }
    }
  }
  __syncthreads();  // keys final, histogram readers done
  block_compact<NW>(keys, n, n_sink, n_local, prefix, mask, r, off, members, out, stride,
                    count_out, out_lds, count_lds, red);
}

// Select for one segment: `sc` points at its n scores, `keys` / `hist` at
// this wave's LDS (cap_keys + 256 words). Writes out[0..stride) and *count_out.
__device__ __forceinline__ void wave_select(uint32_t* __restrict__ keys, uint32_t* __restrict__ hist,
                                            int cap_keys, const float* __restrict__ sc, int n, int k,
                                            int n_sink, int n_local, int mode, uint32_t rnd_word,
                                            int32_t* __restrict__ out, int stride,
                                            int32_t* __restrict__ count_out, int lane) {
  using namespace topk_detail;
  n = n > cap_keys ? cap_keys : n;  // a wrong host max_pages must not overrun LDS
  // Load the segment 8 elements per lane at a time (all loads in flight).
  for (int base = 0; base < n; base += 64 * kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + 64 * u + lane;
      v[u] = i < n ? sc[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + 64 * u + lane;
      if (i < n) keys[i] = (i < n_sink || i >= n - n_local) ? 0u : score_key(v[u]);
    }
  }
  wave_sync();
  wave_select_keys(keys, hist, n, k, n_sink, n_local, mode, rnd_word, out, stride, count_out, lane);
}

}  // namespace vx
