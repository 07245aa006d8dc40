// Radix top-k over one (sequence, KV head) segment of page scores.
//
// Vortex paper note, "System design > 1. vFlow": keep the top-k blocks by
// score; "System design > 3. Execution backend": top-k is the indexer's
// bottleneck, served by a radix top-k with an approximate mode (stochastic
// early termination and remapping) when recall can be traded for time.
//
// Scores become order-preserving 32-bit keys in LDS (forced pages get key 0
// and never compete). The selection rule has one answer: the forced pages
// plus the kk best candidates by (score desc, page index asc).
//
// Register select (segments of up to 256 keys, one wave): each lane holds
// its keys in registers and a threshold tau is searched two bits per step,
// most significant first: per step, three ballot counts (one ballot per key
// register) tell how many keys reach each of the three candidate values, so
// no LDS round trip or barrier is needed, and the search stops as soon as
// exactly kk keys reach tau. Keys above tau are taken, and the first
// kk - count(> tau) keys equal to tau in index order; a ballot + mbcnt
// compaction writes the survivors in ascending page order. The approximate
// mode first maps the candidates' scores affinely onto 256 buckets (the
// remap) and runs the same search over the 9-bit bucket codes only (the
// early termination); the places left in the boundary bucket are filled
// cyclically from a random offset (the stochastic part).
//
// Block select (longer segments, exact mode, small k): every wave selects
// the local top kk of a contiguous range of the keys in registers; the
// union of the local lists holds the global top kk (a key outside its
// range's top kk has kk better keys in the same order), so one wave then
// selects from at most NW * kk candidates the same way. Otherwise (large k,
// very long segments, approximate mode) the block runs 8-bit digit passes:
// LDS histograms shared by the waves, a DPP wave scan to find the digit, an
// early exit when the boundary bucket is exactly needed, then an ordered
// compaction by all waves.
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

// Number of the wave's register keys >= t (R registers, the first ru used).
// ru and t must be wave-uniform (they are kept in scalar registers, so the
// loop has no divergent branch and the count stays scalar).
template <int R>
__device__ __forceinline__ uint32_t count_ge(const uint32_t (&kv)[R], int ru, uint32_t t) {
  uint32_t c = 0;
#pragma unroll
  for (int u = 0; u < R; ++u)
    if (u < ru) c += (uint32_t)__popcll(__ballot(kv[u] >= t));
  return __builtin_amdgcn_readfirstlane(c);
}

// A threshold for the kk best of the wave's register keys (1 <= kk <= number
// of nonzero keys, keys below 2^(top+1), top odd): the largest tau with
// count_ge(tau) >= kk, decided two bits per step from the top (three
// independent counts per step), or an earlier tau with count_ge(tau) == kk
// exactly, where the keys >= tau already are the kk best. Either way the
// kk best are the keys > tau plus the first kk - count_ge(tau + 1) keys
// equal to tau.
template <int R>
__device__ __forceinline__ uint32_t select_threshold(const uint32_t (&kv)[R], int ru, uint32_t kk,
                                                     int top) {
  ru = __builtin_amdgcn_readfirstlane(ru);
  kk = __builtin_amdgcn_readfirstlane(kk);
  uint32_t tau = 0;
  for (int bit = __builtin_amdgcn_readfirstlane(top) - 1; bit >= 0; bit -= 2) {
    const uint32_t t1 = tau | (1u << bit), t2 = tau | (2u << bit), t3 = tau | (3u << bit);
    const uint32_t c1 = count_ge<R>(kv, ru, t1);
    const uint32_t c2 = count_ge<R>(kv, ru, t2);
    const uint32_t c3 = count_ge<R>(kv, ru, t3);
    uint32_t c;
    if (c3 >= kk) { tau = t3; c = c3; }
    else if (c2 >= kk) { tau = t2; c = c2; }
    else if (c1 >= kk) { tau = t1; c = c1; }
    else { c = 0; }
    if (c == kk) break;
  }
  return __builtin_amdgcn_readfirstlane(tau);
}

// Ordered compaction from registers: lane key u is element i0 + 64 u + lane
// (code 0 = not a candidate). Survivors: forced pages (i < n_sink or
// i >= n - n_local), codes > tau, and r of the codes == tau taken in index
// order cyclically from offset `off` over their `members`. Writes
// out[o0 + rank] (global) and out_lds[o0 + rank] (each nullable); returns the
// number written.
template <int R>
__device__ __forceinline__ uint32_t reg_compact(const uint32_t (&code)[R], const int32_t (&idx)[R],
                                                int ru, int n, int n_sink, int n_local,
                                                uint32_t tau, uint32_t r, uint32_t off,
                                                uint32_t members, int32_t* __restrict__ out,
                                                int32_t* __restrict__ out_lds, uint32_t o0) {
  ru = __builtin_amdgcn_readfirstlane(ru);
  tau = __builtin_amdgcn_readfirstlane(tau);
  r = __builtin_amdgcn_readfirstlane(r);
  off = __builtin_amdgcn_readfirstlane(off);
  members = __builtin_amdgcn_readfirstlane(members);
  uint32_t written = __builtin_amdgcn_readfirstlane(o0), tie_seen = 0;
  // r == 0 or r == members: every tie is dropped or every tie taken, no ranks needed
  const bool ranked = r != 0 && r < members;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (u >= ru) break;
    const int i = idx[u];
    const bool forced = i >= 0 && i < n && (i < n_sink || i >= n - n_local);
    const bool above = code[u] > tau;
    const bool tie = code[u] != 0u && code[u] == tau;
    bool take = forced || above || (tie && r != 0);
    if (ranked) {
      const unsigned long long tmask = __ballot(tie);
      const uint32_t trank = tie_seen + rank_below(tmask);
      tie_seen += (uint32_t)__popcll(tmask);
      // cyclic position from off: trank, off < members, so one wrap at most
      uint32_t pos = trank + members - off;
      pos = pos >= members ? pos - members : pos;
      take = forced || above || (tie && pos < r);
    }
    const unsigned long long smask = __ballot(take);
    if (take) {
      if (out) out[written + rank_below(smask)] = i;
      if (out_lds) out_lds[written + rank_below(smask)] = i;
    }
    written += (uint32_t)__popcll(smask);
  }
  return written - o0;
}

// Register select of one segment of n <= 64 R keys by one wave (see the top
// of the file). keys: the segment's keys in LDS.
template <int R>
__device__ __forceinline__ void wave_select_reg(const uint32_t* __restrict__ keys, int n, int k,
                                                int n_sink, int n_local, int mode,
                                                uint32_t rnd_word, int32_t* __restrict__ out,
                                                int stride, int32_t* __restrict__ count_out,
                                                int lane, int32_t* __restrict__ out_lds,
                                                int32_t* __restrict__ count_lds) {
  n = __builtin_amdgcn_readfirstlane(min(n, 64 * R));
  k = __builtin_amdgcn_readfirstlane(k);
  n_sink = __builtin_amdgcn_readfirstlane(n_sink);
  n_local = __builtin_amdgcn_readfirstlane(n_local);
  mode = __builtin_amdgcn_readfirstlane(mode);
  const int nf = min(n, n_sink + n_local);  // forced: a prefix and a suffix of [0, n)
  const int nc = n - nf;
  const int kk = min(k, nc);
  constexpr int ru = R;  // keys past n are 0: below every threshold, never counted
  uint32_t code[R];
  int32_t idx[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int i = 64 * u + lane;
    idx[u] = i;
    code[u] = i < n ? keys[i] : 0u;
  }
  // Defaults: kk == nc takes every candidate (codes > 0), kk == 0 none.
  uint32_t tau = kk == nc ? 0u : 0xffffffffu, r = 0, off = 0, members = 0;
  if (kk > 0 && kk < nc) {
    int top = 31;  // odd: two bits per search step
    if (mode == VX_TOPK_APPROX) {
      // remap: candidates' scores onto 256 buckets, code = bucket + 1
      uint32_t kmax = 0u, kminc = 0u;  // kminc: max of ~key, so min = ~kminc
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (code[u]) { kmax = max(kmax, code[u]); kminc = max(kminc, ~code[u]); }
      const float mx = key_score(wave_max(kmax)), mn = key_score(~wave_max(kminc));
      const float wdt = __fsub_rn(mx, mn);
      const bool spread = wdt > 0.f;
      const float inv = spread ? __fdiv_rn(256.f, wdt) : 0.f;
#pragma unroll
      for (int u = 0; u < R; ++u) {
        if (code[u]) {
          uint32_t bk = 0;
          if (spread) {
            const float t = floorf(__fmul_rn(__fsub_rn(key_score(code[u]), mn), inv));
            bk = t >= 255.f ? 255u : (uint32_t)t;
          }
          code[u] = bk + 1u;
        }
      }
      top = 9;
    }
    tau = select_threshold<R>(code, ru, (uint32_t)kk, top);
    const uint32_t above = count_ge<R>(code, ru, tau + 1u);
    members = count_ge<R>(code, ru, tau) - above;
    r = (uint32_t)kk - above;
    off = (mode == VX_TOPK_APPROX && members) ? rnd_word % members : 0u;
  }
  const uint32_t total = reg_compact<R>(code, idx, ru, n, n_sink, n_local, tau, r, off, members,
                                        out, out_lds, 0u);
  if (out)
    for (int i = (int)total + lane; i < stride; i += 64) out[i] = -1;
  if (lane == 0) {
    if (count_out) *count_out = (int32_t)total;
    if (count_lds) *count_lds = (int32_t)total;
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

// Select for one segment of n <= kBlockSelectMin keys already in this
// wave's LDS (keys[i] = 0 for a forced page, else score_key of its score).
// Writes out[0..stride) and *count_out, and, when given, the chosen ids to
// out_lds[0..count) and the count to *count_lds.
__device__ __forceinline__ void wave_select_keys(const uint32_t* __restrict__ keys, int n, int k,
                                                 int n_sink, int n_local, int mode,
                                                 uint32_t rnd_word, int32_t* __restrict__ out,
                                                 int stride, int32_t* __restrict__ count_out,
                                                 int lane, int32_t* __restrict__ out_lds = nullptr,
                                                 int32_t* __restrict__ count_lds = nullptr) {
  static_assert(kBlockSelectMin == 256, "four register keys per lane");
  topk_detail::wave_select_reg<4>(keys, n, k, n_sink, n_local, mode, rnd_word, out, stride,
                                  count_out, lane, out_lds, count_lds);
}

// The last step of the block selects, by one wave: kk of the nsl <= 64 R2
// candidate ids cand[0 .. nsl) (LDS, ascending page index, -1 = no
// candidate; their keys are nonzero and at least kk of them) are selected by
// the register select; the forced prefix [0, ns) and suffix [ss, n) frame
// them in the output.
template <int R2>
__device__ __forceinline__ void final_select(const uint32_t* __restrict__ keys,
                                             const int32_t* __restrict__ cand, int nsl, int n,
                                             int kk, int n_sink, int n_local,
                                             int32_t* __restrict__ out, int stride,
                                             int32_t* __restrict__ count_out,
                                             int32_t* __restrict__ out_lds,
                                             int32_t* __restrict__ count_lds, int lane) {
  using namespace topk_detail;
  const int nf = min(n, n_sink + n_local);
  const int ru2 = R2 <= 4 ? R2 : (nsl + 63) / 64;
  uint32_t cv[R2];
  int32_t cx[R2];
#pragma unroll
  for (int u = 0; u < R2; ++u) {
    const int j = 64 * u + lane;
    const int id = (u < ru2 && j < nsl) ? cand[j] : -1;
    cx[u] = id;
    cv[u] = id >= 0 ? keys[id] : 0u;
  }
  const uint32_t tau2 = select_threshold<R2>(cv, ru2, (uint32_t)kk, 31);
  const uint32_t above2 = count_ge<R2>(cv, ru2, tau2 + 1u);
  const uint32_t mem2 = count_ge<R2>(cv, ru2, tau2) - above2;
  const int ns = min(n_sink, n), ss = max(ns, n - n_local);
  reg_compact<R2>(cv, cx, ru2, n, 0, 0, tau2, (uint32_t)kk - above2, 0u, mem2, out, out_lds,
                  (uint32_t)ns);
  for (int i = lane; i < ns; i += 64) {
    if (out) out[i] = i;
    if (out_lds) out_lds[i] = i;
  }
  for (int i = ss + lane; i < n; i += 64) {
    const int o = ns + kk + (i - ss);
    if (out) out[o] = i;
    if (out_lds) out_lds[o] = i;
  }
  const int total = nf + kk;
  if (out)
    for (int i = total + lane; i < stride; i += 64) out[i] = -1;
  if (lane == 0) {
    if (count_out) *count_out = (int32_t)total;
    if (count_lds) *count_lds = (int32_t)total;
  }
}

// Exact block select by local top-kk lists (see the top of the file): wave
// w selects the kk best keys of its range of ceil(n / NW) <= 64 R1 keys, then
// wave 0 selects kk of the NW kk <= 64 R2 candidates. hist: LDS for the
// candidate ids. Called by every thread with 0 < kk < the candidate count.
template <int NW, int R1, int R2>
__device__ __forceinline__ void block_union_select(const uint32_t* __restrict__ keys,
                                                   uint32_t* __restrict__ hist, int n, int kk,
                                                   int n_sink, int n_local,
                                                   int32_t* __restrict__ out, int stride,
                                                   int32_t* __restrict__ count_out,
                                                   int32_t* __restrict__ out_lds,
                                                   int32_t* __restrict__ count_lds) {
  using namespace topk_detail;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int per = (n + NW - 1) / NW;
  // Local top kk of wave w's range [lo, hi): candidate ids to cand[w kk ..
  // (w + 1) kk), in index order, -1 after the last.
  int32_t* cand = (int32_t*)hist;
  const int lo = min(n, w * per), hi = min(n, lo + per);
  const int ru1 = R1 <= 2 ? R1 : (hi - lo + 63) / 64;  // keys past hi are 0, never counted
  uint32_t kv[R1];
  int32_t ix[R1];
#pragma unroll
  for (int u = 0; u < R1; ++u) {
    const int i = lo + 64 * u + lane;
    ix[u] = i;
    kv[u] = (u < ru1 && i < hi) ? keys[i] : 0u;
  }
  uint32_t tau = 0, rr = 0, mem = 0;  // fewer than kk candidates: take them all
  if (count_ge<R1>(kv, ru1, 1u) > (uint32_t)kk) {
    tau = select_threshold<R1>(kv, ru1, (uint32_t)kk, 31);
    const uint32_t above = count_ge<R1>(kv, ru1, tau + 1u);
    mem = count_ge<R1>(kv, ru1, tau) - above;
    rr = (uint32_t)kk - above;
  }
  const uint32_t c = reg_compact<R1>(kv, ix, ru1, n, 0, 0, tau, rr, 0u, mem, nullptr,
                                     cand + w * kk, 0u);
  for (int j = (int)c + lane; j < kk; j += 64) cand[w * kk + j] = -1;
  __syncthreads();
  if (w != 0) return;
  final_select<R2>(keys, cand, NW * kk, n, kk, n_sink, n_local, out, stride, count_out, out_lds,
                   count_lds, lane);
}

// Exact block select by a lower bound (see the top of the file): wave w
// takes the q = ceil(kk / NW) largest keys of its range of ceil(n / NW) <=
// 64 R1 keys by q rounds of wave max (each round takes every key equal to
// the maximum, so ties count fully) and reports the smallest taken, T_w, and
// how many it took, c_w. Every key >= min_w T_w is a survivor: at least
// sum_w c_w keys reach that bound, so when that sum is >= kk the kk-th
// largest key does too, and the survivors hold the whole selection,
// boundary ties included. The survivors' ids go to hist in index order and
// one wave selects kk of them. Returns false, after a barrier and with
// nothing written, when the bound does not hold (some ranges hold fewer than
// q candidates) or more than 256 keys survive; the caller then selects
// another way. red: 2 NW words; hist: kSelectHistWords words. Called by
// every thread with 0 < kk < the candidate count and q <= kMaxBoundRounds.
constexpr int kMaxBoundRounds = 8;
template <int NW, int R1>
__device__ __forceinline__ bool block_bounded_select(const uint32_t* __restrict__ keys,
                                                     uint32_t* __restrict__ hist,
                                                     uint32_t* __restrict__ red, int n, int kk,
                                                     int n_sink, int n_local,
                                                     int32_t* __restrict__ out, int stride,
                                                     int32_t* __restrict__ count_out,
                                                     int32_t* __restrict__ out_lds,
                                                     int32_t* __restrict__ count_lds) {
  using namespace topk_detail;
  static_assert(NW <= 16, "survivor counts at the end of hist");
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int per = (n + NW - 1) / NW;
  const int lo = min(n, w * per), hi = min(n, lo + per);
  const int ru1 = R1 <= 2 ? R1 : (hi - lo + 63) / 64;  // keys past hi are 0
  uint32_t kv[R1], work[R1];
  int32_t ix[R1];
#pragma unroll
  for (int u = 0; u < R1; ++u) {
    const int i = lo + 64 * u + lane;
    ix[u] = i;
    kv[u] = (u < ru1 && i < hi) ? keys[i] : 0u;
    work[u] = kv[u];
  }
  const int q = (kk + NW - 1) / NW;
  uint32_t taken = 0, tw = 0;
  for (int round = 0; round < q; ++round) {
    uint32_t lm = 0u;
#pragma unroll
    for (int u = 0; u < R1; ++u)
      if (u < ru1) lm = max(lm, work[u]);
    const uint32_t v = wave_max(lm);
    if (v == 0u) break;  // no key left in the range
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < R1; ++u) {
      if (u < ru1) {
        const bool e = work[u] == v;
        c += (uint32_t)__popcll(__ballot(e));
        work[u] = e ? 0u : work[u];
      }
    }
    taken += __builtin_amdgcn_readfirstlane(c);
    tw = v;
    if (taken >= (uint32_t)q) break;
  }
  if (lane == 0) {
    red[w] = tw;
    red[NW + w] = taken;
  }
  __syncthreads();
  const uint32_t cw = lane < NW ? red[NW + lane] : 0u;
  const uint32_t tl = lane < NW ? red[lane] : 0u;
  const uint32_t bound = ~wave_max(cw ? ~tl : 0u);  // min of T_w over ranges that took keys
  const uint32_t reach = __builtin_amdgcn_readlane(prefix_sum(cw), 63);
  const uint32_t mine = count_ge<R1>(kv, ru1, bound);
  uint32_t* scount = hist + kSelectHistWords - 16;
  if (lane == 0) scount[w] = mine;
  __syncthreads();
  const uint32_t sv = lane < NW ? scount[lane] : 0u;
  const uint32_t pre = prefix_sum(sv);
  const uint32_t S = __builtin_amdgcn_readlane(pre, 63);
  const uint32_t off = __builtin_amdgcn_readlane(pre - sv, w);
  if (reach < (uint32_t)kk || S > 256u) {  // the same decision in every wave
    __syncthreads();  // every wave is done with red and hist
    return false;
  }
  int32_t* cand = (int32_t*)hist;
  reg_compact<R1>(kv, ix, ru1, n, 0, 0, bound - 1u, 0u, 0u, 0u, nullptr, cand, off);
  __syncthreads();
  if (w != 0) return true;
  if (S <= 64u)
    final_select<1>(keys, cand, (int)S, n, kk, n_sink, n_local, out, stride, count_out, out_lds,
                    count_lds, lane);
  else
    final_select<4>(keys, cand, (int)S, n, kk, n_sink, n_local, out, stride, count_out, out_lds,
                    count_lds, lane);
  return true;
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
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  n = __builtin_amdgcn_readfirstlane(n);
  k = __builtin_amdgcn_readfirstlane(k);
  n_sink = __builtin_amdgcn_readfirstlane(n_sink);
  n_local = __builtin_amdgcn_readfirstlane(n_local);
  mode = __builtin_amdgcn_readfirstlane(mode);
  const int nf = min(n, n_sink + n_local);
  const int nc = n - nf;
  const int kk = min(k, nc);
  const int per = (n + NW - 1) / NW;
  if (mode == VX_TOPK_EXACT && kk > 0 && kk < nc && per <= 512 &&
      (kk + NW - 1) / NW <= kMaxBoundRounds) {
    const bool done =
        per <= 128 ? block_bounded_select<NW, 2>(keys, hist, red, n, kk, n_sink, n_local, out,
                                                 stride, count_out, out_lds, count_lds)
                   : block_bounded_select<NW, 8>(keys, hist, red, n, kk, n_sink, n_local, out,
                                                 stride, count_out, out_lds, count_lds);
    if (done) return;
  }
  if (mode == VX_TOPK_EXACT && kk > 0 && kk < nc && per <= 512 && NW * kk <= kSelectHistWords) {
    if (per <= 128 && NW * kk <= 256)
      block_union_select<NW, 2, 4>(keys, hist, n, kk, n_sink, n_local, out, stride, count_out,
                                   out_lds, count_lds);
    else
      block_union_select<NW, 8, kSelectHistWords / 64>(keys, hist, n, kk, n_sink, n_local, out,
                                                       stride, count_out, out_lds, count_lds);
    return;
  }
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

// Select for one segment: `sc` points at its n scores, `keys` at this
// wave's LDS (cap_keys words, cap_keys <= kBlockSelectMin). Writes
// out[0..stride) and *count_out.
__device__ __forceinline__ void wave_select(uint32_t* __restrict__ keys, int cap_keys,
                                            const float* __restrict__ sc, int n, int k, int n_sink,
                                            int n_local, int mode, uint32_t rnd_word,
                                            int32_t* __restrict__ out, int stride,
                                            int32_t* __restrict__ count_out, int lane) {
  using namespace topk_detail;
  n = n > cap_keys ? cap_keys : n;  // a wrong host max_pages must not overrun LDS
  float v[kBlockSelectMin / 64];
#pragma unroll
  for (int u = 0; u < kBlockSelectMin / 64; ++u) {
    const int i = 64 * u + lane;
    v[u] = i < n ? sc[i] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < kBlockSelectMin / 64; ++u) {
    const int i = 64 * u + lane;
    if (i < n) keys[i] = (i < n_sink || i >= n - n_local) ? 0u : score_key(v[u]);
  }
  wave_sync();
  wave_select_keys(keys, n, k, n_sink, n_local, mode, rnd_word, out, stride, count_out, lane);
}

}  // namespace vx
