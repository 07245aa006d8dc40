// MLA geometry: one 576-wide latent stream (512 latent + 64 rope columns)
// shared by every query head; values are the first 512 columns of each row.
//
// Vortex paper note, "Key results > MLA": the rope part matters for routing,
// so pages are scored on all 576 columns; "System design > 3. Execution
// backend" adds an attention kernel for general MLA geometry. The scoring
// and attention here are dense bf16 contractions across the query heads on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// MFMA operand layout used throughout (lane l, 16 = l % 16, q4 = l / 16):
//   A (16 x 32):  lane holds row (l % 16), k elements 8*q4 .. 8*q4+7
//   B (32 x 16):  lane holds column (l % 16), the same k elements
//   D (16 x 16):  lane holds rows 4*q4 + i (i < 4), column (l % 16)
// A and B read the k elements from the same offsets, so the contraction is
// exact whatever order the hardware sums them in.
#include "topk_wave.h"

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
// The centroid of sequence b's newest page (page n - 1, its valid tokens
// among L): thread t < DK / 4 sums columns 4t .. 4t+3 over the tokens in
// order, all of its loads in flight at once, divides once (IEEE), and writes
// the fp32 centroid, its bf16 copy and that copy to `row` (LDS).
__device__ __forceinline__ void mla_newest_centroid(const Meta& m, const uint16_t* __restrict__ kp,
                                                    float* __restrict__ cent32,
                                                    uint16_t* __restrict__ cent, int b, int n,
                                                    int L, uint16_t* __restrict__ row) {
  constexpr int kQuads = DK / 4;  // 4-column groups of a key row
  const int t = threadIdx.x;
  const int P = m.page_size;
  const int nv = min(P, L - (n - 1) * P);
  const int pid = phys_page(m, m.indptr[b] + n - 1);
  if (t < kQuads) {
    const uint16_t* kb = kp + (size_t)pid * P * DK + 4 * t;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    for (int t0 = 0; t0 < nv; t0 += 64) {
      uint2 x[64];
      // Loads past the last token repeat it (never added), so no load has a
      // condition: one mask per load would not fit the scalar registers.
#pragma unroll
      for (int u = 0; u < 64; ++u) x[u] = *(const uint2*)(kb + (size_t)min(t0 + u, nv - 1) * DK);
      // every load issued before the first add (the scheduler would
      // otherwise interleave them and wait for each load in turn)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 64; ++u)
        if (t0 + u < nv) {
          s0 += bf16_lo(x[u].x); s1 += bf16_hi(x[u].x);
          s2 += bf16_lo(x[u].y); s3 += bf16_hi(x[u].y);
        }
    }
    const float fn = (float)nv;
    const float c0 = s0 / fn, c1 = s1 / fn, c2 = s2 / fn, c3 = s3 / fn;
    const size_t o = (size_t)pid * DK + 4 * t;
    *(float4*)(cent32 + o) = make_float4(c0, c1, c2, c3);
    const uint2 h = make_uint2((uint32_t)f32_to_bf16(c0) | ((uint32_t)f32_to_bf16(c1) << 16),
                               (uint32_t)f32_to_bf16(c2) | ((uint32_t)f32_to_bf16(c3) << 16));
    *(uint2*)(cent + o) = h;
    *(uint2*)(row + 4 * t) = h;
  }
}

// Score partial of this lane's page column: the 16 MT query rows staged in
// LDS (qs) times the lane's centroid slice bf, summed over the rows and the
// lane group; lanes of one column hold the same sum.
template <int MT, int KS>
__device__ __forceinline__ float mla_column_score(const uint16_t* __restrict__ qs,
                                                  const u32x4 (&bf)[KS], int lane) {
  const int col = lane & 15, q4 = lane >> 4;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* arow = qs + (16 * mt + col) * ROW + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma(*(const u32x4*)(arow + 32 * ks), bf[ks], acc[mt]);
  }
  float sc = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) sc += (acc[mt][0] + acc[mt][1]) + (acc[mt][2] + acc[mt][3]);
  sc += __shfl_xor(sc, 16);
  sc += __shfl_xor(sc, 32);
  return sc;
}

// grid (ceil(max_pages / 64) [+ 1 with refresh], B), 4 waves; the blocks
// are renumbered XCD-major into (x, sequence b) below. Scoring block x: wave
// w scores the 16 pages [64 x + 16 w, +16) of sequence b;
// each lane loads its page id and centroid slice before the query rows are
// staged, so the block waits on two dependent loads, not three. With
// `refresh`, the last block of each row instead recomputes the sequence's
// newest page centroid (fp32 and its bf16 copy) from its keys, in token
// order with one IEEE divide per column (the cache stage's arithmetic), and
// scores that page from the new bf16 row in LDS; the scoring blocks skip
// it. The per-page arithmetic is the same in both kinds of block.
template <int MT, int KS>
__global__ __launch_bounds__(256) void scores_mla_kernel(Meta m, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ kp,
                                                         float* __restrict__ cent32,
                                                         uint16_t* __restrict__ cent, int refresh,
                                                         float scale, float* __restrict__ scores) {
  constexpr int kQPer = (16 * MT * (DK / 8) + 255) / 256;  // query vectors per thread
  constexpr int kQuads = DK / 4;                           // 4-column groups of a key row
  static_assert(kQuads <= 256, "the refresh takes one 4-column group per thread");
  __shared__ __attribute__((aligned(16))) uint16_t qs[16 * MT * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t newrow[DK];
  // A sequence's blocks on one XCD (its 37 KB of query rows fetched once
  // there, not by all eight), its refresh block (the longest) dispatched
  // first among them.
  const int vb = xcd_major(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int b = vb / gridDim.x, bx = gridDim.x - 1 - vb % gridDim.x;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int col = lane & 15, q4 = lane >> 4;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  int n = (L + m.page_size - 1) / m.page_size;
  n = n > cap ? cap : n;
  const bool refresh_block = refresh && bx == gridDim.x - 1;
  const int n_scored = refresh ? n - 1 : n;  // pages the scoring blocks take
  const int blk0 = bx * 64;
  if (refresh_block ? n == 0 : blk0 >= n_scored) return;  // whole block: no barrier reached

  // This sequence's query rows (16 * MT heads x 576), loaded now, stored in LDS below.
  const uint16_t* qb = q + (size_t)b * (16 * MT) * DK;
  u32x4 qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int c = t + 256 * u;
    if (c < 16 * MT * (DK / 8)) qv[u] = *(const u32x4*)(qb + (c / (DK / 8)) * DK + 8 * (c % (DK / 8)));
  }
  // This lane's page and its centroid slice (B operand: page col, 8 columns per k step).
  const int p = refresh_block ? n - 1 : blk0 + 16 * w + col;
  const bool valid = refresh_block ? col == 0 && w == 0 : p < n_scored;
  u32x4 bf[KS];  // KS k steps of 32 columns: 18 = all 576, 16 = the 512 latent ones
  if (!refresh_block) {
    const uint16_t* crow = cent + (size_t)(valid ? phys_page(m, row0 + p) : 0) * DK + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bf[ks] = valid ? *(const u32x4*)(crow + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  } else {
    mla_newest_centroid(m, kp, cent32, cent, b, n, L, newrow);
  }
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int c = t + 256 * u;
    if (c < 16 * MT * (DK / 8)) *(u32x4*)(qs + (c / (DK / 8)) * ROW + 8 * (c % (DK / 8))) = qv[u];
  }
  __syncthreads();
  if (refresh_block) {
    if (w != 0) return;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bf[ks] = valid ? *(const u32x4*)(newrow + 8 * q4 + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  } else if (blk0 + 16 * w >= n_scored) {
    return;
  }

  const float sc = mla_column_score<MT, KS>(qs, bf, lane);
  if (lane < 16 && valid) scores[row0 + p] = sc * scale;
}

// ---------------------------------------------------------------- attention
// One block of 4 MT waves (MT head tiles of 16) per (sequence b, split s);
// the split holds an even share of the selection's entries, consumed one
// 64-token page (a "chunk") at a time. Wave w works on head tile mt = w / 4
// and quarter u = w % 4: token tile u (tokens 16 u ..) in q.k^T, value
// columns 128 u .. 128 u + 127 in P.V.
//
// Staging: every chunk goes straight from HBM into LDS with direct loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16 * lane)
// through a ring of two chunk slots, so the next chunk streams in while the
// current one is consumed and no register holds staging data. A slot is 72
// wave-wide 1 KB loads; the lane -> (token t, 16-byte granule g) map of each
// load is chosen so that both MFMA operand reads below hit distinct 16-byte
// bank groups within every 8 and every 16 lanes:
//   latent granule g < 64:  load 16 (g / 16) + t / 4,
//                           lane 16 (t % 4) + ((g ^ t) % 16);
//   rope granule g >= 64:   load 64 + t / 8,
//                           lane 8 (t % 8) + (((g - 64) ^ t) % 8).
// q.k^T  v_mfma_f32_16x16x32_bf16, A = the tile's query rows (registers),
//        B = key granules (lane: token l % 16, 8 columns per k step).
// P.V    lane (q4, c) reads tokens 8 q4 .. 8 q4 + 7 of each 32-token half,
//        columns 8 c .. 8 c + 7 of its quarter (eight 16-byte reads); taking
//        N-tile e's columns as {8 c + e}, element e of the lane's eight rows
//        is its B fragment (byte permutes); P, bf16 through LDS, is the A
//        operand.
// Softmax: probabilities are taken against a per-row reference maximum that
// moves only when some logit of a chunk exceeds it by more than kLazy (log2
// units); below that, probabilities up to 2^kLazy are used as they are. The
// waves raise a flag in LDS when they see such a logit; only then (and
// always at the first chunk) are the chunk's row maxima exchanged, the
// accumulators rescaled and P recomputed. Each lane sums the probabilities
// of its own token; the sums are reduced once, at the end.
constexpr int CHT = 64;                   // tokens per chunk (one page)
constexpr int kChunkLoads = CHT * DK / 8 / 64;   // 72 wave-wide 16-byte loads
constexpr int kCpolNT = 2;  // cache-policy operand of the direct loads: non-temporal
constexpr int kSlotBytes = kChunkLoads * 1024;
constexpr int PROW = CHT + 8;             // padded P row (bf16), 144 B
constexpr float kLazy = 8.f;
static_assert(DV == 4 * 128, "four 128-column value quarters");

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32, round to nearest even
}

// B fragment e of P.V: element e of each of the lane's eight value rows.
__device__ __forceinline__ u32x4 column_frag(const u32x4* v, int e) {
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  auto word = [&](const u32x4& x) {
    return (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  };
  u32x4 r;
  r.x = __builtin_amdgcn_perm(word(v[1]), word(v[0]), sel);
  r.y = __builtin_amdgcn_perm(word(v[3]), word(v[2]), sel);
  r.z = __builtin_amdgcn_perm(word(v[5]), word(v[4]), sel);
  r.w = __builtin_amdgcn_perm(word(v[7]), word(v[6]), sel);
  return r;
}

typedef __attribute__((address_space(3))) void lds_void;

// Block barrier for LDS data only. __syncthreads() would also wait for the
// direct loads in flight into the other slot (they write LDS); here only this
// wave's own LDS reads and writes are completed (lgkmcnt 0) before the
// barrier, and the signal fences keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS of the attention part. The two slots are separate arrays: the
// compiler then sees that reads of one slot do not depend on direct loads
// still in flight into the other.
#define VX_MLA_ATTN_LDS(MT)                                              \
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kSlotBytes];   \
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kSlotBytes];   \
  __shared__ __attribute__((aligned(16))) uint16_t pl[16 * (MT) * PROW]; \
  __shared__ float rmax[4][16 * (MT)];                                   \
  __shared__ int flag[4 * (MT)];                                         \
  __shared__ int pg_phys[kMaxPagesPerSplit];                             \
  __shared__ int pg_nv[kMaxPagesPerSplit];

// Entries [p0, p1) of the selection's stride belong to split s of S.
__device__ __forceinline__ void mla_split(int stride, int s, int S, int& p0, int& p1) {
  p0 = (int)(((long)stride * s) / S);
  p1 = min((int)(((long)stride * (s + 1)) / S), p0 + kMaxPagesPerSplit);
}

// Attention of sequence b's query heads over the np pages listed in
// pg_phys / pg_nv (LDS, visible to the block); split s of S. Called by
// every thread of the block.
template <int MT>
__device__ __forceinline__ void mla_attend(uint8_t* slot0, uint8_t* slot1, uint16_t* pl,
                                           float (*rmax)[16 * MT], int* flag, const int* pg_phys,
                                           const int* pg_nv, int np, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ kp, int b, int s, int S,
                                           float qscale, float* __restrict__ out,
                                           float* __restrict__ lse, float* __restrict__ part_o,
                                           float* __restrict__ part_ml) {
  constexpr int HQ = 16 * MT;
  constexpr int NW = 4 * MT;
  constexpr int LPW = kChunkLoads / NW;  // loads per wave per chunk
  static_assert(kChunkLoads % NW == 0 && 64 % NW == 0, "loads split evenly");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int mt = w >> 2, u = w & 3;
  const int col = lane & 15, q4 = lane >> 4;

  // query rows 16 mt + col, columns 32 ks + 8 q4 .. +7
  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = q + ((size_t)b * HQ + 16 * mt + col) * DK + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *(const u32x4*)(qrow + 32 * ks);
  }

  // Per-lane parts of the slot layout (see above).
  // Direct loads w + NW k: latent load i (< 64) fetches token 4 (i % 16) + lane / 16,
  // granule 16 (i / 16) + ((lane ^ t) % 16); t % 16 depends on i only through i % 4 = w % 4.
  const int src_lat = (lane >> 4) * DK + 8 * ((lane ^ (4 * (w & 3) + (lane >> 4))) & 15);
  const int src_rope = (lane >> 3) * DK + 8 * (64 + ((lane ^ (lane >> 3)) & 7));
  // q.k^T reads: token 16 u + col, granule 4 ks + q4.
  int qk_off[6];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
    qk_off[k4] = (4 * u + (col >> 2)) * 1024 + (16 * (col & 3) + (((4 * k4 + q4) ^ col) & 15)) * 16;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
    qk_off[4 + k2] = (64 + 2 * u + (col >> 3)) * 1024 + (8 * (col & 7) + (((4 * k2 + q4) ^ col) & 7)) * 16;
  // P.V reads: token 32 kb + 8 q4 + r, granule 16 u + col.
  int pv_off[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
    pv_off[r] = (16 * u + 2 * q4 + (r >> 2)) * 1024 + (16 * (r & 3) + ((col ^ (8 * (q4 & 1) + r)) & 15)) * 16;

  f32x4 o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { mrow[i] = kNegBig; lrow[i] = 0.f; }

  // This wave's loads w + NW k of chunk c, straight into its slot.
  auto issue = [&](int c, uint8_t* slot_c) {
    const uint16_t* page = kp + (size_t)__builtin_amdgcn_readfirstlane(pg_phys[c]) * CHT * DK;
    uint8_t* slot = slot_c + 1024 * w;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int i = w + NW * k;
      const int off = k < 64 / NW ? 4 * (i & 15) * DK + 128 * (i >> 4) + src_lat
                                  : 8 * (i - 64) * DK + src_rope;
      // cache policy nt: each page is read once per step
      __builtin_amdgcn_global_load_lds((const void*)(page + off), (lds_void*)(slot + 1024 * NW * k),
                                       16, 0, kCpolNT);
    }
  };
  // Chunk c: consumed from `slot`; chunk c + 1 streams into `other`.
  // `first` (a literal at each call) is chunk 0.
  auto chunk = [&](int c, const uint8_t* slot, uint8_t* other, bool first) {
    // Wait for this wave's loads of chunk c (nothing else is in flight
    // here: vmcnt 0); the barrier then makes every wave's share visible and
    // ends every read of chunk c - 1, whose slot chunk c + 1 takes; then
    // chunk c + 1 is issued and streams in while chunk c is computed. Chunk 0
    // goes out alone, so every block's first page comes back before the
    // second pages are requested (both at once ran 0.5 us slower).
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    if (first)
      barrier_lds();  // (A): nothing but LDS to wait for once vmcnt is 0
    else
      __syncthreads();  // (A)
    if (c + 1 < np) issue(c + 1, other);
    const int nv = pg_nv[c];

    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int off = ks < 16 ? qk_off[ks & 3] + (ks >> 2) * 16384 : qk_off[4 + (ks - 16)];
      sacc = mfma(qf[ks], *(const u32x4*)(slot + off), sacc);
    }
    const bool tok_ok = 16 * u + col < nv;
    // Probabilities against the current reference maxima; a wave that sees
    // a logit above its row's reference + kLazy raises the block's flag.
    float z[4], p[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = tok_ok ? sacc[i] * qscale : -INFINITY;
      need = need || z[i] > mrow[i] + kLazy;
      p[i] = __builtin_amdgcn_exp2f(z[i] - mrow[i]);
    }
    const bool wave_need = __ballot(need) != 0;
    if (lane == 0) flag[w] = wave_need ? 1 : 0;
    auto write_p = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pl[(16 * mt + 4 * q4 + i) * PROW + 16 * u + col] = (uint16_t)bf16_bits(p[i]);
    };
    write_p();
    barrier_lds();  // (B) P and the flags of the whole chunk in LDS
    int any = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) any |= flag[v];
    if (any) {
      // Rare (always at the first chunk): move every row's reference to
      // max(reference, chunk maximum), rescale, recompute P. The flags are
      // the same for every wave, so the whole block takes this branch.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mx = group_max<16>(z[i]);
        if (col == 0) rmax[u][16 * mt + 4 * q4 + i] = mx;
      }
      barrier_lds();
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * q4 + i;
        const float mx = fmaxf(fmaxf(rmax[0][r], rmax[1][r]), fmaxf(rmax[2][r], rmax[3][r]));
        const float mref = fmaxf(mrow[i], mx);
        alpha[i] = __builtin_amdgcn_exp2f(mrow[i] - mref);
        mrow[i] = mref;
        p[i] = __builtin_amdgcn_exp2f(z[i] - mref);
        lrow[i] *= alpha[i];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[e][i] *= alpha[i];
      write_p();
      barrier_lds();  // P rewritten; every wave has read the flags and maxima
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[i] += p[i];  // this lane's token; summed at the end

#pragma unroll
    for (int kb = 0; kb < CHT / 32; ++kb) {
      u32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = *(const u32x4*)(slot + pv_off[r] + 8192 * kb);
      if (nv < CHT) {  // rows past the page's valid tokens hold no data: make them zero
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (32 * kb + 8 * q4 + r >= nv) v[r] = u32x4{0u, 0u, 0u, 0u};
      }
      const u32x4 pa = *(const u32x4*)(pl + (16 * mt + col) * PROW + 32 * kb + 8 * q4);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = mfma(pa, column_frag(v, e), o[e]);
    }
  };

  // Chunk 0 is computed before the loop: a loop entry waits for every load
  // in flight (the query rows loaded above are used inside it), which there
  // is chunk 1 only, needed next anyway.
  if (np > 0) {
    issue(0, slot0);
    chunk(0, slot0, slot1, true);
  }
  for (int c = 1; c < np; c += 2) {
    chunk(c, slot1, slot0, false);
    if (c + 1 < np) chunk(c + 1, slot0, slot1, false);
  }

  // Row sums: over the 16 tokens of the lane group, then the four token tiles.
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = group_sum<16>(lrow[i]);
  __syncthreads();
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rmax[u][16 * mt + 4 * q4 + i] = lrow[i];
  }
  __syncthreads();

  // results: rows 16 mt + 4 q4 + i, columns 128 u + 8 col + e
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 16 * mt + 4 * q4 + i;
    const float l = (rmax[0][head] + rmax[1][head]) + (rmax[2][head] + rmax[3][head]);
    const int d0 = 128 * u + 8 * col;
    if (S == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* dst = out + ((size_t)b * HQ + head) * DV + d0;
      *(float4*)dst = make_float4(o[0][i] * inv, o[1][i] * inv, o[2][i] * inv, o[3][i] * inv);
      *(float4*)(dst + 4) = make_float4(o[4][i] * inv, o[5][i] * inv, o[6][i] * inv, o[7][i] * inv);
      if (lse && u == 0 && col == 0)
        lse[(size_t)b * HQ + head] = l > 0.f ? (mrow[i] + log2f(l)) * kLn2 : -INFINITY;
    } else {
      // The split's partial rows go through slot0 (no chunk is in flight or
      // read any more), stored below as whole rows.
      float* tile = (float*)slot0;
      *(f32x4*)(tile + head * DV + d0) = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]};
      *(f32x4*)(tile + head * DV + d0 + 4) = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]};
      if (u == 0 && col == 0) {
        const size_t ps = ((size_t)b * HQ + head) * S + s;
        part_ml[2 * ps] = mrow[i];
        part_ml[2 * ps + 1] = l;
      }
    }
  }
  if (S > 1) {
    // Non-temporal stores (the partials are read once, by the merge, and a
    // kernel's end then has no dirty L2 lines of them to write back), each
    // covering 1 KB of a row: from the registers' layout (8 columns per
    // lane, lanes 32 B apart) every store would fill half lines, which the
    // memory then writes twice (21.6 against 14.7 MB per step).
    static_assert(16 * MT * DV * 4 <= kSlotBytes, "the partial rows fit in a slot");
    __syncthreads();
    const float* tile = (const float*)slot0;
    for (int c = t; c < HQ * DV / 4; c += 64 * NW) {
      const int head = c / (DV / 4), d = 4 * (c % (DV / 4));
      __builtin_nontemporal_store(*(const f32x4*)(tile + head * DV + d),
                                  (f32x4*)(part_o + (((size_t)b * HQ + head) * S + s) * DV + d));
    }
  }
}

// Attention over a selection made by the caller (sel / sel_count).
template <int MT>
__global__ __launch_bounds__(256 * MT) void attn_mla_kernel(
    Meta m, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
    const int32_t* __restrict__ sel, int stride, const int32_t* __restrict__ sel_count,
    float qscale, int S, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  VX_MLA_ATTN_LDS(MT)
  static_assert(kMaxPagesPerSplit <= 256 * MT, "one page-list entry per thread");
  const int t = threadIdx.x;
  const int s = blockIdx.x % S, b = blockIdx.x / S;
  // The split is over the stride, not the count, so the split's entries load
  // together with the count instead of after it; entries at or past the
  // count are dropped.
  int p0, p1;
  mla_split(stride, s, S, p0, p1);
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  const int count = cap > 0 ? min(sel_count[b], stride) : 0;
  const int np = max(0, min(p1, count) - p0);
  // m.page_size == CHT (checked on the host): one chunk per page
  if (t < p1 - p0) {
    int lp = sel[(size_t)b * stride + p0 + t];
    if (t < np) {
      lp = lp < 0 ? 0 : (lp >= cap ? cap - 1 : lp);
      pg_phys[t] = phys_page(m, row0 + lp);
      pg_nv[t] = max(0, min(CHT, L - lp * CHT));
    }
  }
  __syncthreads();  // page list ready
  mla_attend<MT>(slot0, slot1, pl, rmax, flag, pg_phys, pg_nv, np, q, kp, b, s, S, qscale, out,
                 lse, part_o, part_ml);
}

// Selection and attention in one kernel (the decode step after scoring):
// every split block of sequence b selects b's pages from its scores itself
// (the same radix top-k as the top-k kernels, so the same selection), block
// s == 0 writes sel / sel_count, and each block attends over its split's
// share. The keys and the selected ids use the chunk slots before any
// chunk is loaded.
struct MlaStepArgs {
  Meta m;
  const uint16_t* q;
  const uint16_t* kp;
  const float* scores;
  int k, n_sink, n_local, mode;
  const uint32_t* rnd;
  int32_t* sel;
  int stride;
  int32_t* sel_count;
  float qscale;
  int S;
  float* out;
  float* lse;
  float* part_o;
  float* part_ml;
  int cap_keys;
  // Newest-page refresh in blocks B * S .. B * S + B - 1 (refresh_blocks):
  // only when the newest page is forced, so its score is not needed by the
  // selections read meanwhile.
  int refresh_blocks;
  float* cent32;
  uint16_t* cent;
  float score_scale;
  float* scores_w;  // = scores
};

// The refresh the scorer's last block does (mla_newest_centroid, then that
// page's score from the new bf16 row), for sequence b by a whole block of
// the step kernel: qs and row are LDS (the attention's slots, unused here).
template <int MT, int KS>
__device__ __forceinline__ void mla_step_refresh(const MlaStepArgs& a, int b, uint16_t* qs,
                                                 uint16_t* row) {
  const Meta& m = a.m;
  const int t = threadIdx.x, lane = t & 63;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  const int n = min((L + m.page_size - 1) / m.page_size, cap);
  if (n == 0) return;  // whole block: no barrier reached
  const uint16_t* qb = a.q + (size_t)b * (16 * MT) * DK;
  for (int c = t; c < 16 * MT * (DK / 8); c += blockDim.x)
    *(u32x4*)(qs + (c / (DK / 8)) * ROW + 8 * (c % (DK / 8))) =
        *(const u32x4*)(qb + (c / (DK / 8)) * DK + 8 * (c % (DK / 8)));
  mla_newest_centroid(m, a.kp, a.cent32, a.cent, b, n, L, row);
  __syncthreads();
  if (t >= 64) return;
  const int col = lane & 15, q4 = lane >> 4;
  u32x4 bf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bf[ks] = col == 0 ? *(const u32x4*)(row + 8 * q4 + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  const float sc = mla_column_score<MT, KS>(qs, bf, lane);
  if (lane == 0) a.scores_w[row0 + n - 1] = sc * a.score_scale;
}

template <int MT, int KS>
__global__ __launch_bounds__(256 * MT) void decode_mla_kernel(MlaStepArgs a) {
  VX_MLA_ATTN_LDS(MT)
  __shared__ int32_t cnt_l;
  constexpr int NW = 4 * MT;
  static_assert(kMaxPagesPerSplit <= 256 * MT, "one page-list entry per thread");
  static_assert(DK / 4 <= 256 * MT, "the refresh takes one 4-column group per thread");
  static_assert(16 * MT * ROW * 2 <= kSlotBytes, "the refresh stages the query rows in a slot");
  if ((int)blockIdx.x >= a.m.batch * a.S) {  // whole block
    mla_step_refresh<MT, KS>(a, blockIdx.x - a.m.batch * a.S, (uint16_t*)slot0, (uint16_t*)slot1);
    return;
  }
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int s = blockIdx.x % a.S, b = blockIdx.x / a.S;
  const Meta& m = a.m;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = seq_len_clamped(m, b);
  const int n = min(min((L + CHT - 1) / CHT, cap), a.cap_keys);
  uint32_t* keys = (uint32_t*)slot0;  // cap_keys + kSelectExtraWords words
  int32_t* sel_l = (int32_t*)slot1;   // the selection, ascending
  // The physical page of every entry, loaded together with the scores when
  // it fits in slot1 after the selection's stride: the page list then needs
  // no global load after the select.
  const int pid_off = (a.stride + 63) / 64 * 64;
  const bool pid_in_lds = (size_t)(pid_off + n) * 4 <= (size_t)kSlotBytes;
  int32_t* pid_l = sel_l + pid_off;
  for (int i = t; i < n; i += 64 * NW) {
    keys[i] = (i < a.n_sink || i >= n - a.n_local) ? 0u : topk_detail::score_key(a.scores[row0 + i]);
    if (pid_in_lds) pid_l[i] = phys_page(m, row0 + i);
  }
  __syncthreads();
  const uint32_t rnd = a.mode == VX_TOPK_APPROX ? a.rnd[b] : 0u;
  int32_t* gsel = s == 0 ? a.sel + (size_t)b * a.stride : nullptr;
  int32_t* gcnt = s == 0 ? a.sel_count + b : nullptr;
  if (n > kBlockSelectMin)
    block_select_keys<NW>(keys, keys + a.cap_keys, keys + a.cap_keys + kSelectHistWords, n, a.k, a.n_sink,
                          a.n_local, a.mode, rnd, gsel, a.stride, gcnt, sel_l, &cnt_l);
  else if (w == 0)
    wave_select_keys(keys, n, a.k, a.n_sink, a.n_local, a.mode, rnd, gsel,
                     a.stride, gcnt, lane, sel_l, &cnt_l);
  __syncthreads();  // selection in LDS
  int p0, p1;
  mla_split(a.stride, s, a.S, p0, p1);
  const int count = min(cnt_l, a.stride);
  const int np = max(0, min(p1, count) - p0);
  if (t < np) {
    const int lp = sel_l[p0 + t];
    pg_phys[t] = pid_in_lds ? pid_l[lp] : phys_page(m, row0 + lp);
    pg_nv[t] = max(0, min(CHT, L - lp * CHT));
  }
  __syncthreads();  // page list ready; keys and selection no longer read
  mla_attend<MT>(slot0, slot1, pl, rmax, flag, pg_phys, pg_nv, np, a.q, a.kp, b, s, a.S, a.qscale,
                 a.out, a.lse, a.part_o, a.part_ml);
}

}  // namespace

hipError_t launch_scores_mla_sized(const Meta& m, const vx_geom& g, const void* q,
                                   const void* k_pool, float* cent32, uint16_t* cent_bf16,
                                   int refresh, float scale, float* scores, int max_pages,
                                   hipStream_t s) {
  if (m.nnz == 0 || m.batch == 0) return hipSuccess;
  dim3 grid((max_pages + 63) / 64 + (refresh ? 1 : 0), m.batch), block(256);
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

bool decode_step_mla_fusable(int max_pages, int sel_stride) {
  const int cap_keys = (max_pages + 63) / 64 * 64;
  return (size_t)(cap_keys + kSelectExtraWords) * 4 <= (size_t)kSlotBytes &&
         (size_t)sel_stride * 4 <= (size_t)kSlotBytes;
}

hipError_t launch_decode_step_mla(const Meta& m, const vx_geom& g, const void* q,
                                  const void* k_pool, const float* scores, int k, int n_sink,
                                  int n_local, int mode, const uint32_t* rnd, int32_t* sel,
                                  int sel_stride, int32_t* sel_count, float sm_scale,
                                  int num_splits, float* out, float* lse, float* part_o,
                                  float* part_ml, int max_pages, int refresh, float* cent32,
                                  uint16_t* cent_bf16, float score_scale, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  MlaStepArgs a{};
  a.refresh_blocks = refresh;
  a.cent32 = cent32;
  a.cent = cent_bf16;
  a.score_scale = score_scale;
  a.scores_w = const_cast<float*>(scores);
  a.m = m;
  a.q = (const uint16_t*)q;
  a.kp = (const uint16_t*)k_pool;
  a.scores = scores;
  a.k = k;
  a.n_sink = n_sink;
  a.n_local = n_local;
  a.mode = mode;
  a.rnd = rnd;
  a.sel = sel;
  a.stride = sel_stride;
  a.sel_count = sel_count;
  a.qscale = sm_scale * kLog2e;
  a.S = num_splits;
  a.out = out;
  a.lse = lse;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.cap_keys = (max_pages + 63) / 64 * 64;
  dim3 grid(m.batch * num_splits + (refresh ? m.batch : 0));
  const bool latent_only = g.score_dim == DV;
  if (g.num_q_heads == 32) {
    if (latent_only)
      hipLaunchKernelGGL((decode_mla_kernel<2, DV / 32>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mla_kernel<2, KSTEPS>), grid, dim3(512), 0, s, a);
  } else if (g.num_q_heads == 16) {
    if (latent_only)
      hipLaunchKernelGGL((decode_mla_kernel<1, DV / 32>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mla_kernel<1, KSTEPS>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_mla(const Meta& m, const vx_geom& g, const void* q,
                                const void* k_pool, const int32_t* sel, int sel_stride,
                                const int32_t* sel_count, float sm_scale, int num_splits,
                                int pages_per_split, float* out, float* lse, float* part_o,
                                float* part_ml, hipStream_t s) {
  if (m.batch == 0) return hipSuccess;
  const float qscale = sm_scale * kLog2e;
  dim3 grid(m.batch * num_splits);
  if (g.num_q_heads == 32)
    hipLaunchKernelGGL(attn_mla_kernel<2>, grid, dim3(512), 0, s, m, (const uint16_t*)q,
                       (const uint16_t*)k_pool, sel, sel_stride, sel_count, qscale, num_splits,
                       out, lse, part_o, part_ml);
  else if (g.num_q_heads == 16)
    hipLaunchKernelGGL(attn_mla_kernel<1>, grid, dim3(256), 0, s, m, (const uint16_t*)q,
                       (const uint16_t*)k_pool, sel, sel_stride, sel_count, qscale, num_splits,
                       out, lse, part_o, part_ml);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vx
