// Indexer, GQA geometry: page scoring, optionally fused with the cache
// stage's refresh of each sequence's newest page.
//
// Vortex paper note, "System design > 1. vFlow": the indexer multiplies the
// query with the cached centroids; "System design > 3. Execution backend":
// sequence-local operators are fused. One kernel runs
//   1. cache refresh: the page holding a sequence's newest token gets its
//      centroid recomputed from its keys (fp32 sum in token order, one IEEE
//      divide: the same bits as the cache-stage kernels) and stored back;
//      the wave that scores that page does it, so no other block waits;
//   2. scoring: a GQA group's query heads share their KV head's pages, so the
//      group's heads are summed first and each page costs one fp32 dot
//      product per KV head; the kernel streams every centroid row once.
// The top-k runs as the next kernel: making one block wait for the scores of
// others needs device-scope release/acquire fences, which on this chip write
// back and invalidate the whole L2 of the compute die, far dearer than a
// launch boundary.
//
// Mapping: the grid runs over page-table entries (no block idles past a
// short sequence's end). A block of kWaves waves covers kWaves * kPPW
// consecutive entries; it sums the query of the sequence owning its first
// entry once into LDS. Each wave finds its entries' sequences with a ballot
// over a window of indptr, loading all its centroid rows before using any. A
// row [Hkv][Dk] fp32 is read as 16-byte chunks, chunk c = i*64 + lane, so
// every load instruction covers 1 KB contiguous; chunk c belongs to head
// c / (Dk/4), whose Dk/4 lanes reduce with DPP row ops. CB16: the rows are
// the centroids' bf16 copy, chunk c being its 8 bytes of the same 4 dims,
// scored with the same arithmetic on the bf16 values.
#include "vx_internal.h"

namespace vx {
namespace {

constexpr int kPPW = 4;    // pages per wave, all rows in flight at once
constexpr int kWaves = 8;  // waves per block
constexpr int kSpan = kWaves * kPPW;    // entries per block

template <typename T>
__device__ __forceinline__ float4 load4(const T* p) { return Quad<T>::widen(Quad<T>::load(p)); }

struct IndexArgs {
  Meta m;
  int hq, hkv;
  const void* q;
  const void* kp;         // key pool (refresh only)
  float* cent;            // [pool][Hkv][Dk] fp32
  uint16_t* cent_bf16;    // optional bf16 copy (refresh writes it)
  int refresh;            // recompute the newest page of every sequence first
  float scale;
  float* scores;          // [Hkv][nnz]
};

// Scaled group sum of the query of sequence b for the 4 dims of chunk c
// (head c / W of the KV heads): sum over the group's heads in head order.
template <typename QT, int DK, int GG>
__device__ __forceinline__ float4 group_query(const QT* q, int hq, int G, int b, int c,
                                              float scale) {
  constexpr int W = DK / 4;
  const int g = c / W, d = (c % W) * 4;
  const QT* qb = q + ((size_t)b * hq + (size_t)g * G) * DK + d;
  float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (GG > 0) {
    typename Quad<QT>::raw x[GG];
#pragma unroll
    for (int h = 0; h < GG; ++h) x[h] = Quad<QT>::load(qb + (size_t)h * DK);
#pragma unroll
    for (int h = 0; h < GG; ++h) {
      const float4 v = Quad<QT>::widen(x[h]);
      s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
    }
  } else {
    for (int h = 0; h < G; ++h) {
      const float4 v = load4(qb + (size_t)h * DK);
      s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
    }
  }
  return make_float4(s4.x * scale, s4.y * scale, s4.z * scale, s4.w * scale);
}

// Score of the head owning chunk c: the chunk's 4 products, then a sum over
// the W lanes of the head. Written by the head's first lane.
template <int W>
__device__ __forceinline__ void score_chunk(float4 qs, float4 r, bool ok, int c, size_t nnz, int j,
                                            float* scores) {
  float sc = qs.x * r.x;
  sc = fmaf(qs.y, r.y, sc);
  sc = fmaf(qs.z, r.z, sc);
  sc = fmaf(qs.w, r.w, sc);
  sc = group_sum<W>(sc);
  if (ok && (c % W) == 0) scores[(size_t)(c / W) * nnz + j] = sc;
}

// QT: query type; KV: key type; R: 16-byte chunks per lane per row;
// GG > 0: group size known at compile time; FULL: every lane owns a chunk of
// every row load (Hkv * Dk / 4 == R * 64).
//
// Phases: (a) every wave loads its pages' rows and finds their sequences;
// (b) it scores them, except, when refreshing, each sequence's newest page,
// which it lists in LDS; (c) the listed pages are refreshed by R waves each
// (wave w % R takes chunk group w % R, so a row's chunks load in parallel
// and every lane has up to 32 tokens in flight) and scored from the fresh
// values with the same arithmetic as (b).
template <typename QT, typename KV, int DK, int R, int GG, bool FULL, bool CB16>
__global__ __launch_bounds__(64 * kWaves) void index_gqa_kernel(IndexArgs a) {
  constexpr int W = DK / 4;
  __shared__ float4 qsum[R * 64];  // the block's first sequence's scaled query sum
  __shared__ int n_new;            // newest pages listed by phase (b)
  __shared__ int new_j[kSpan], new_b[kSpan];

  const Meta& m = a.m;
  const QT* q = (const QT*)a.q;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nchunk = a.hkv * DK / 4;
  const int G = GG > 0 ? GG : a.hq / a.hkv;
  const int P = m.page_size;
  const int j_blk = blockIdx.x * kSpan;
  const int j0 = j_blk + w * kPPW;
  const bool active = j0 < m.nnz;
  const int nj = active ? min(kPPW, m.nnz - j0) : 0;
  if (threadIdx.x == 0) n_new = 0;

  // (a) Two independent chains of two round trips each: page ids -> centroid
  // rows, and the block's first sequence -> windows of indptr / seq_lens and
  // the query rows.
  const int my_pid = active ? phys_page(m, j0 + min(lane, nj - 1)) : 0;
  const int b_blk = __builtin_amdgcn_readfirstlane(wave_find_seq(m.indptr, m.batch, j_blk, lane));
  float4 rows[kPPW][R];
  if (active) {
#pragma unroll
    for (int u = 0; u < kPPW; ++u) {
      const size_t row = (size_t)__builtin_amdgcn_readlane(my_pid, u) * a.hkv * DK;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int ch = i * 64 + lane;
        const bool in = FULL || ch < nchunk;
        // centroid rows are streamed once per step: non-temporal loads
        if constexpr (CB16) {
          const u32x2 raw = in ? __builtin_nontemporal_load((const u32x2*)(a.cent_bf16 + row) + ch)
                               : u32x2{0u, 0u};
          rows[u][i] = make_float4(bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y));
        } else {
          const u32x4 raw = in ? __builtin_nontemporal_load((const u32x4*)(a.cent + row) + ch)
                               : u32x4{0u, 0u, 0u, 0u};
          rows[u][i] = make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y),
                                   __uint_as_float(raw.z), __uint_as_float(raw.w));
        }
      }
    }
  }
  // lane i: start and length of sequence b_blk + i
  const int wnd = m.indptr[min(b_blk + lane, m.batch)];
  const int wlen = m.seq_lens[min(b_blk + lane, m.batch - 1)];
  for (int c = threadIdx.x; c < R * 64; c += 64 * kWaves)
    qsum[c] = c < nchunk ? group_query<QT, DK, GG>(q, a.hq, G, b_blk, c, a.scale)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
  // The sequence of each page: b_blk plus the number of later window starts
  // at or before the entry (one ballot); past a run of 62 sequences without
  // entries, the search and scalar loads.
  int bq[kPPW];
  bool valid[kPPW], newest[kPPW];
#pragma unroll
  for (int u = 0; u < kPPW; ++u) {
    const int j = min(j0 + u, m.nnz - 1);
    const int c = __popcll(__ballot(lane >= 1 && wnd <= j));
    int b, s0, s1, L;
    if (c < 63) {
      b = b_blk + c;
      s0 = __builtin_amdgcn_readlane(wnd, c);
      s1 = __builtin_amdgcn_readlane(wnd, c + 1);
      L = __builtin_amdgcn_readlane(wlen, c);
    } else {
      b = __builtin_amdgcn_readfirstlane(wave_find_seq(m.indptr, m.batch, j, lane));
      s0 = m.indptr[b];
      s1 = m.indptr[b + 1];
      L = m.seq_lens[b];
    }
    const int cap = s1 - s0;
    L = min(max(L, 0), cap * P);
    const int np = min((L + P - 1) / P, cap);
    const int p = j0 + u - s0;
    bq[u] = b;
    valid[u] = u < nj && p < np;
    newest[u] = valid[u] && p == np - 1;
  }
  __syncthreads();  // query sums ready, list cleared

  // (b) scores of the rows already loaded, one pass per distinct sequence
  uint32_t todo = 0;
#pragma unroll
  for (int u = 0; u < kPPW; ++u) {
    const bool later = a.refresh && newest[u];
    todo |= (valid[u] && !later) ? (1u << u) : 0u;
    if (later && lane == 0) {
      const int k = atomicAdd(&n_new, 1);
      new_j[k] = j0 + u;
      new_b[k] = bq[u];
    }
  }
  while (todo) {
    const int ufirst = __builtin_ctz(todo);
    int b = 0;
#pragma unroll
    for (int u = 0; u < kPPW; ++u) b = u == ufirst ? bq[u] : b;
    float4 qs[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = i * 64 + lane;
      if (b == b_blk) qs[i] = qsum[c];
      else qs[i] = (FULL || c < nchunk) ? group_query<QT, DK, GG>(q, a.hq, G, b, c, a.scale)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kPPW; ++u) {
      if (((todo >> u) & 1u) && bq[u] == b) {
        todo &= ~(1u << u);
#pragma unroll
        for (int i = 0; i < R; ++i)
          score_chunk<W>(qs[i], rows[u][i], FULL || i * 64 + lane < nchunk, i * 64 + lane, m.nnz,
                         j0 + u, a.scores);
      }
    }
  }
  if (!a.refresh) return;

  // (c) refresh and score the listed newest pages
  __syncthreads();
  constexpr int kTok = sizeof(KV) == 2 ? 32 : 16;  // tokens in flight per lane
  const int i = w % R;
  const int c = i * 64 + lane;
  const bool own = FULL || c < nchunk;
  const int total = n_new;
  for (int k = w / R; k < total; k += kWaves / R) {
    const int j = new_j[k], b = new_b[k];
    const int p = j - m.indptr[b];
    const int nv = min(P, seq_len_clamped(m, b) - p * P);
    const int pid = phys_page(m, j);
    const int g = c / W, d = (c % W) * 4;
    const KV* col = (const KV*)a.kp + ((size_t)pid * a.hkv + g) * P * DK + d;
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t0 = 0; t0 < nv; t0 += kTok) {
      typename Quad<KV>::raw x[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t)
        if (own && t0 + t < nv) x[t] = Quad<KV>::load(col + (size_t)(t0 + t) * DK);
#pragma unroll
      for (int t = 0; t < kTok; ++t)
        if (own && t0 + t < nv) {
          const float4 v = Quad<KV>::widen(x[t]);
          s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
        }
    }
    const float fn = (float)nv;
    const float4 c4 = make_float4(s4.x / fn, s4.y / fn, s4.z / fn, s4.w / fn);
    if (own) {
      const size_t o = (size_t)pid * a.hkv * DK + 4 * c;
      *(float4*)(a.cent + o) = c4;
      if (a.cent_bf16) {
        const uint32_t lo = (uint32_t)f32_to_bf16(c4.x) | ((uint32_t)f32_to_bf16(c4.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(c4.z) | ((uint32_t)f32_to_bf16(c4.w) << 16);
        *(uint2*)(a.cent_bf16 + o) = make_uint2(lo, hi);
      }
    }
    float4 qs;
    if (b == b_blk) qs = qsum[c];
    else qs = own ? group_query<QT, DK, GG>(q, a.hq, G, b, c, a.scale) : make_float4(0.f, 0.f, 0.f, 0.f);
    // CB16: the page is scored from the copy's value, the bf16 rounding
    const float4 cs =
        CB16 ? make_float4(bf16_to_f32(f32_to_bf16(c4.x)), bf16_to_f32(f32_to_bf16(c4.y)),
                           bf16_to_f32(f32_to_bf16(c4.z)), bf16_to_f32(f32_to_bf16(c4.w)))
             : c4;
    score_chunk<W>(qs, cs, own, c, m.nnz, j, a.scores);
  }
}

template <typename QT, typename KV, int DK, int R, bool FULL, bool CB16>
hipError_t launch_r(const IndexArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  dim3 grid((a.m.nnz + kSpan - 1) / kSpan), block(64 * kWaves);
#define VX_IX(GG) \
  hipLaunchKernelGGL((index_gqa_kernel<QT, KV, DK, R, GG, FULL, CB16>), grid, block, 0, s, a)
  switch (G) {
    case 1: VX_IX(1); break;
    case 2: VX_IX(2); break;
    case 4: VX_IX(4); break;
    case 8: VX_IX(8); break;
    default: VX_IX(0); break;
  }
#undef VX_IX
  return hipGetLastError();
}

template <typename QT, typename KV, int DK, bool CB16 = false>
hipError_t launch_dk(const IndexArgs& a, hipStream_t s) {
  const int nchunk = a.hkv * DK / 4;
  if (nchunk <= 64)
    return nchunk == 64 ? launch_r<QT, KV, DK, 1, true, CB16>(a, s)
                        : launch_r<QT, KV, DK, 1, false, CB16>(a, s);
  if (nchunk <= 128)
    return nchunk == 128 ? launch_r<QT, KV, DK, 2, true, CB16>(a, s)
                         : launch_r<QT, KV, DK, 2, false, CB16>(a, s);
  if (nchunk <= 256)
    return nchunk == 256 ? launch_r<QT, KV, DK, 4, true, CB16>(a, s)
                         : launch_r<QT, KV, DK, 4, false, CB16>(a, s);
  return nchunk == 512 ? launch_r<QT, KV, DK, 8, true, CB16>(a, s)
                       : launch_r<QT, KV, DK, 8, false, CB16>(a, s);
}

}  // namespace

hipError_t launch_scores_gqa(const Meta& m, const vx_geom& g, const void* q, const void* k_pool,
                             float* cent, uint16_t* cent_bf16, int refresh, float scale,
                             float* scores, hipStream_t s) {
  if (m.nnz == 0 || m.batch == 0) return hipSuccess;
  IndexArgs a{};
  a.m = m;
  a.hq = g.num_q_heads;
  a.hkv = g.num_kv_heads;
  a.q = q;
  a.kp = k_pool;
  a.cent = cent;
  a.cent_bf16 = cent_bf16;
  a.refresh = refresh;
  a.scale = scale;
  a.scores = scores;
  const bool f32 = g.kv_dtype == VX_F32;  // the bf16 copy is scored with bf16 keys only
  if (g.head_dim_k == 64)
    return f32 ? launch_dk<float, float, 64>(a, s)
               : g.score_bf16 ? launch_dk<uint16_t, uint16_t, 64, true>(a, s)
                              : launch_dk<uint16_t, uint16_t, 64>(a, s);
  return f32 ? launch_dk<float, float, 128>(a, s)
             : g.score_bf16 ? launch_dk<uint16_t, uint16_t, 128, true>(a, s)
                            : launch_dk<uint16_t, uint16_t, 128>(a, s);
}

}  // namespace vx
