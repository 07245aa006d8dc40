// Indexer selection: per-(sequence, KV head) radix top-k over page scores.
//
// Vortex paper note, "System design > 1. vFlow": keep the top-k blocks by
// score; "System design > 3. Execution backend": top-k is the indexer's
// bottleneck, served by a radix top-k with an approximate mode (stochastic
// early termination and remapping) when recall can be traded for time.
//
// One wave per segment. Scores become order-preserving 32-bit keys in LDS
// (forced pages get key 0 and never compete). Exact mode runs up to four
// 8-bit digit passes, most significant first: an LDS histogram of the digit
// among keys that still match the chosen prefix, a suffix scan across the
// wave to find the digit where the count from the top reaches the remaining
// need r, and an early exit when that bucket holds exactly r keys. The
// survivors are then compacted in index order with ballot + mbcnt prefix
// sums, which yields ascending page ids and the lower-index tie-break.
// Approximate mode maps candidate scores affinely onto 256 buckets, runs one
// pass and fills the r remaining places from the boundary bucket cyclically
// from a random offset.
#include "vx_internal.h"

namespace vx {
namespace {

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

// Suffix scan over lanes: lane l gets sum_{l' >= l} x(l').
__device__ __forceinline__ uint32_t suffix_scan(uint32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
  return x;
}

struct Digit {
  uint32_t d;      // chosen bucket
  uint32_t above;  // keys strictly above it (among those matching the prefix)
  uint32_t count;  // keys inside it
};

// Find the bucket where the count from the top first reaches r (1 <= r <= total).
__device__ __forceinline__ Digit find_digit(const uint32_t* hist, uint32_t r, int lane) {
  const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
  const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const uint32_t incl = suffix_scan(h0 + h1 + h2 + h3, lane);  // S(4 lane)
  const uint32_t s0 = incl, s1 = incl - h0, s2 = s1 - h1, s3 = s2 - h2;  // S(4 lane + i)
  int hit = -1;
  uint32_t hab = 0, hcnt = 0;
  if (s3 >= r && s3 - h3 < r) { hit = 3; hab = s3 - h3; hcnt = h3; }
  else if (s2 >= r && s2 - h2 < r) { hit = 2; hab = s2 - h2; hcnt = h2; }
  else if (s1 >= r && s1 - h1 < r) { hit = 1; hab = s1 - h1; hcnt = h1; }
  else if (s0 >= r && s0 - h0 < r) { hit = 0; hab = s0 - h0; hcnt = h0; }
  const unsigned long long found = __ballot(hit >= 0);
  const int src = __ffsll((long long)found) - 1;
  Digit out;
  out.d = (uint32_t)__shfl(4 * lane + hit, src);
  out.above = (uint32_t)__shfl((int)hab, src);
  out.count = (uint32_t)__shfl((int)hcnt, src);
  return out;
}

__global__ __launch_bounds__(256) void topk_kernel(Meta m, int hkv, const float* __restrict__ scores,
                                                   int k, int n_sink, int n_local, int mode,
                                                   const uint32_t* __restrict__ rnd,
                                                   int32_t* __restrict__ sel, int stride,
                                                   int32_t* __restrict__ sel_count, int cap_keys) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int seg = blockIdx.x * (blockDim.x >> 6) + w;
  if (seg >= m.batch * hkv) return;  // whole wave; no block barrier below
  uint32_t* keys = lds + w * (cap_keys + 256);
  uint32_t* hist = keys + cap_keys;

  const int b = seg / hkv, g = seg % hkv;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  int n = (seq_len_clamped(m, b) + m.page_size - 1) / m.page_size;
  n = n > cap ? cap : n;
  n = n > cap_keys ? cap_keys : n;  // a wrong host max_pages must not overrun LDS
  const int nf = min(n, n_sink + n_local);  // forced: a prefix and a suffix of [0, n)
  const int nc = n - nf;
  const int kk = min(k, nc);
  const float* sc = scores + (size_t)g * m.nnz + row0;
  int32_t* out = sel + (size_t)seg * stride;

  for (int i = lane; i < n; i += 64) {
    const bool forced = i < n_sink || i >= n - n_local;
    keys[i] = forced ? 0u : score_key(sc[i]);
  }
  wave_sync();

  // Survivors: candidates with (key & mask) > prefix, plus `r` of those with
  // (key & mask) == prefix taken in index order from offset `off` (cyclic
  // over the `members` of that tie group).
  uint32_t prefix = 0, mask = 0, r = (uint32_t)kk, off = 0, members = (uint32_t)nc;
  if (kk > 0 && kk < nc) {
    if (mode == VX_TOPK_APPROX) {
      uint32_t kmin = 0xffffffffu, kmax = 0u;
      for (int i = lane; i < n; i += 64) {
        const uint32_t kv = keys[i];
        if (kv) { kmin = min(kmin, kv); kmax = max(kmax, kv); }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
      }
      const float mn = key_score(kmin), mx = key_score(kmax);
      const float wdt = __fsub_rn(mx, mn);
      const bool spread = wdt > 0.f;
      const float inv = spread ? __fdiv_rn(256.f, wdt) : 0.f;
      for (int i = lane; i < n; i += 64) {
        const uint32_t kv = keys[i];
        if (kv) {
          uint32_t bk = 0;
          if (spread) {
            const float t = floorf(__fmul_rn(__fsub_rn(key_score(kv), mn), inv));
            bk = t >= 255.f ? 255u : (uint32_t)t;
          }
          keys[i] = (bk << 24) | 1u;  // nonzero; digit 3 is the bucket
        }
      }
      for (int i = lane; i < 256; i += 64) hist[i] = 0;
      wave_sync();
      for (int i = lane; i < n; i += 64) {
        const uint32_t kv = keys[i];
        if (kv) atomicAdd(&hist[kv >> 24], 1u);
      }
      wave_sync();
      const Digit dg = find_digit(hist, r, lane);
      prefix = dg.d << 24;
      mask = 0xff000000u;
      r -= dg.above;
      members = dg.count;
      off = members ? rnd[seg] % members : 0u;
    } else {
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = lane; i < 256; i += 64) hist[i] = 0;
        wave_sync();
        for (int i = lane; i < n; i += 64) {
          const uint32_t kv = keys[i];
          if (kv && (kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
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

  // Ordered compaction (ascending page index).
  uint32_t written = 0, tie_seen = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const bool in = i < n;
    const uint32_t kv = in ? keys[i] : 0u;
    const bool forced = in && (i < n_sink || i >= n - n_local);
    const bool cand = kv != 0u;
    const bool above = cand && (kv & mask) > prefix;
    const bool tie = cand && (kv & mask) == prefix;
    const unsigned long long tmask = __ballot(tie);
    const uint32_t trank = tie_seen + rank_below(tmask);
    tie_seen += (uint32_t)__popcll(tmask);
    bool take = forced || above;
    if (tie && members) take = take || ((trank + members - off) % members) < r;
    const unsigned long long smask = __ballot(take);
    if (take) out[written + rank_below(smask)] = i;
    written += (uint32_t)__popcll(smask);
  }
  for (int i = (int)written + lane; i < stride; i += 64) out[i] = -1;
  if (lane == 0) sel_count[seg] = (int32_t)written;
}

}  // namespace

hipError_t launch_topk_sized(const Meta& m, int hkv, const float* scores, int k, int n_sink,
                             int n_local, int mode, const uint32_t* rand_u32, int32_t* sel,
                             int sel_stride, int32_t* sel_count, int max_pages,
                             int waves_per_block, hipStream_t s) {
  const int segs = m.batch * hkv;
  if (segs == 0) return hipSuccess;
  const int cap_keys = ((max_pages + 63) / 64) * 64;
  const size_t lds = (size_t)waves_per_block * (cap_keys + 256) * sizeof(uint32_t);
  dim3 block(64 * waves_per_block), grid((segs + waves_per_block - 1) / waves_per_block);
  hipLaunchKernelGGL(topk_kernel, grid, block, lds, s, m, hkv, scores, k, n_sink, n_local, mode,
                     rand_u32, sel, sel_stride, sel_count, cap_keys);
  return hipGetLastError();
}

}  // namespace vx
