// Indexer of one (sequence, KV head) segment, GQA geometry: cache refresh of
// the newest page, page scores and the top-k selection, by one block.
//
// Vortex paper note, "System design > 1. vFlow": the indexer multiplies the
// query with the cached centroids and keeps the top-k blocks; "System design
// > 3. Execution backend": sequence-local operators are fused greedily, and
// the radix top-k serves the selection.
//
// Everything the selection needs is local to the segment (sequence b, KV
// head g), so no block waits for another: the block streams the 4*Dk-byte
// slice of head g from every centroid row of b, keeps the scores as radix
// keys in LDS, and its first wave selects from them.
//   - Rows: the waves split b's pages into contiguous ranges; per chunk of
//     kSegChunk load instructions a wave loads the chunk's page ids (one per
//     lane), then all the chunk's row slices (64/W pages per instruction,
//     W = Dk/4 lanes per slice, 16 bytes per lane), all in flight at once.
//   - Scores: the same arithmetic as the flat scorer (group-summed query,
//     4 products per lane, then a W-lane DPP sum), so the bits are equal.
//   - Refresh (optional): the last wave recomputes the newest page's slice
//     from its keys (fp32, token order, one IEEE divide: the cache stage's
//     arithmetic) with up to 32 tokens in flight per lane, writes it back and
//     scores it.
//   - CB16: the rows are read from the bf16 copy of the centroids, 8 bytes
//     per lane for the same 4 dims and the same arithmetic on the bf16
//     values (half the bytes); the refresh scores its page from the bf16
//     rounding of the fresh centroid, the value the copy then holds.
//   - BOUNDS: the Quest-style indexer instead (bounds.h): a head's slice of a
//     page's key bounds is as many bytes as its fp32 centroid slice (bf16
//     minima and maxima, 16 bytes per lane), scored with the stand-alone
//     bound scorer's arithmetic; the refresh recomputes the newest page's
//     bounds.
#pragma once

#include <type_traits>

#include "bounds.h"
#include "topk_wave.h"

namespace vx {

constexpr int kSegChunk = 16;  // row loads in flight per lane

struct SegArgs {
  Meta m;
  int hq, hkv;
  const void* q;
  const void* kp;
  float* cent;
  uint16_t* cent_bf16;
  void* bounds;  // Quest-style indexer: [pool][Hkv][Dk/4][2][4] bf16
  int refresh;
  float scale;
  float* scores;
  int k, n_sink, n_local, mode;
  const uint32_t* rnd;
  int32_t* sel;
  int stride;
  int32_t* sel_count;
  int cap_keys;
  const int32_t* order;  // nullable: order[i] = the sequence block row i serves (whole step)
  int pair_rows;         // > 0: block rows ranked in the kernel and paired (whole step)
  // Append (nullable, centroid indexer with refresh only): the newest token's
  // key and value rows, [B][Hkv][Dk] and [B][Hkv][dv] of the KV type. The
  // refresh then writes both into the token's slot (vp: the value pool) and
  // sums the key from k_new for that slot.
  const void* k_new;
  const void* v_new;
  void* vp;
  int dv;
};

// What the waves other than wave 0 do while wave 0 selects: nothing.
struct NoIdle {
  VX_DEV void operator()(int, int, bool) const {}
};

// The index of segment seg = b * Hkv + g by a block of NW waves (NW <= 16).
// keys: LDS, cap_keys + kSelectExtraWords words (16-byte aligned). pid_lds (nullable, cap_keys ints)
// receives the physical page of every entry in use; sel_lds / count_lds
// (nullable) a copy of the selection. Ends after the selection is written;
// its LDS copies are visible to the block after a barrier. When one wave
// selects (segments of up to kBlockSelectMin pages), that wave calls
// idle(n, L, true) just before its selection and the other waves call
// idle(n, L, false) meanwhile (n pages in use, L tokens; the keys and pid_lds
// are then visible); a longer segment is selected by every wave and idle is
// not called. sel_global == false leaves a.sel / a.sel_count unwritten (the
// caller writes them later from sel_lds / count_lds).
template <typename QT, typename KV, int DK, int GG, int NW, bool BOUNDS = false,
          bool CB16 = false, typename Idle = NoIdle>
VX_DEV void index_segment(const SegArgs& a, int seg, uint32_t* keys, int* pid_lds,
                          int32_t* sel_lds, int32_t* count_lds, Idle idle = Idle{},
                          bool sel_global = true) {
  constexpr int W = DK / 4;    // lanes per row slice
  constexpr int PPI = 64 / W;  // pages per load instruction
  constexpr int kChunk = kSegChunk * PPI;
  static_assert(kChunk <= 64, "one page id per lane");
  static_assert(NW <= 16, "block select reduction words");
  static_assert(!BOUNDS || sizeof(KV) == 2, "bounds slices are 16 bytes per lane for bf16 keys");
  static_assert(!(BOUNDS && CB16), "one page statistic per indexer");

  const Meta& m = a.m;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = seg / a.hkv, g = seg % a.hkv;
  const int P = m.page_size;
  const int row0 = m.indptr[b];
  const int cap = m.indptr[b + 1] - row0;
  const int L = min(max(m.seq_lens[b], 0), cap * P);
  const int n = min(min((L + P - 1) / P, cap), a.cap_keys);
  const int G = GG > 0 ? GG : a.hq / a.hkv;
  const int sub = lane / W, dl = lane % W;

  // Scaled group sum of the query for this lane's 4 dims of head g.
  float4 qs = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    const QT* qb = (const QT*)a.q + ((size_t)b * a.hq + (size_t)g * G) * DK + 4 * dl;
    if constexpr (GG > 0) {
      typename Quad<QT>::raw x[GG];
#pragma unroll
      for (int h = 0; h < GG; ++h) x[h] = Quad<QT>::load(qb + (size_t)h * DK);
#pragma unroll
      for (int h = 0; h < GG; ++h) {
        const float4 v = Quad<QT>::widen(x[h]);
        qs.x += v.x; qs.y += v.y; qs.z += v.z; qs.w += v.w;
      }
    } else {
      for (int h = 0; h < G; ++h) {
        const float4 v = Quad<QT>::widen(Quad<QT>::load(qb + (size_t)h * DK));
        qs.x += v.x; qs.y += v.y; qs.z += v.z; qs.w += v.w;
      }
    }
    qs = make_float4(qs.x * a.scale, qs.y * a.scale, qs.z * a.scale, qs.w * a.scale);
  }
  const bool refresh = a.refresh && n > 0;
  const int nrow = refresh ? n - 1 : n;  // pages scored from their stored rows
  const int rw = refresh ? NW - 1 : NW;
  float* scores = a.scores + (size_t)g * m.nnz + row0;

  // this lane's share of a page's score, from its 16 bytes of the row slice
  auto lane_part = [&](const auto& raw) {
    if constexpr (BOUNDS) {
      float lo[4], hi[4];
      Unit<uint16_t>::widen(raw, lo, hi);
      return unit_bound(qs, lo, hi);
    } else if constexpr (CB16) {
      float sc = qs.x * bf16_lo(raw.x);
      sc = fmaf(qs.y, bf16_hi(raw.x), sc);
      sc = fmaf(qs.z, bf16_lo(raw.y), sc);
      sc = fmaf(qs.w, bf16_hi(raw.y), sc);
      return sc;
    } else {
      float sc = qs.x * __uint_as_float(raw.x);
      sc = fmaf(qs.y, __uint_as_float(raw.y), sc);
      sc = fmaf(qs.z, __uint_as_float(raw.z), sc);
      sc = fmaf(qs.w, __uint_as_float(raw.w), sc);
      return sc;
    }
  };
  auto emit = [&](int p, float part, bool ok) {
    const float sc = group_sum<W>(part);
    if (ok && dl == 0) {
      scores[p] = sc;
      keys[p] = (p < a.n_sink || p >= n - a.n_local) ? 0u : topk_detail::score_key(sc);
    }
  };

  if (w < rw) {
    const int pw0 = (int)(((long)nrow * w) / rw), pw1 = (int)(((long)nrow * (w + 1)) / rw);
    for (int cb = pw0; cb < pw1; cb += kChunk) {
      const bool mine = cb + lane < pw1 && lane < kChunk;
      const int my_pid = mine ? phys_page(m, row0 + cb + lane) : 0;
      if (pid_lds && mine) pid_lds[cb + lane] = my_pid;
      using Slice = std::conditional_t<CB16, u32x2, u32x4>;  // this lane's part of a row
      Slice r[kSegChunk];
#pragma unroll
      for (int t = 0; t < kSegChunk; ++t) {
        const int p = cb + t * PPI + sub;
        const int pid = __shfl(my_pid, t * PPI + sub);
        // rows are streamed once per step: non-temporal loads
        const size_t row = (size_t)pid * a.hkv + g;
        const Slice* src =
            BOUNDS ? (const Slice*)((const uint16_t*)a.bounds + (row * W + dl) * 8)
                   : CB16 ? (const Slice*)(a.cent_bf16 + row * DK + 4 * dl)
                          : (const Slice*)(a.cent + row * DK + 4 * dl);
        r[t] = p < pw1 ? __builtin_nontemporal_load(src) : Slice{};
      }
#pragma unroll
      for (int t = 0; t < kSegChunk; ++t) {
        const int p = cb + t * PPI + sub;
        emit(p, lane_part(r[t]), p < pw1);
      }
    }
  } else if (refresh) {
    // Newest page n-1: lanes 0..W-1 own 4 dims each and sum its tokens in order.
    const int p = n - 1;
    const int nv = min(P, L - p * P);
    const int pid = phys_page(m, row0 + p);
    if (pid_lds && lane == 0) pid_lds[p] = pid;
    const bool own = sub == 0;
    if constexpr (BOUNDS) {
      float part = 0.f;
      if (own) {
        float lo[4], hi[4];
        unit_bounds<uint16_t>((const uint16_t*)a.kp, (uint16_t*)a.bounds, P, a.hkv, DK, pid, nv,
                              g * W + dl, lo, hi);
        part = unit_bound(qs, lo, hi);
      }
      emit(p, part, own);
    } else {
      const KV* col = (const KV*)a.kp + ((size_t)pid * a.hkv + g) * P * DK + 4 * dl;
      constexpr int kTok = sizeof(KV) == 2 ? 32 : 16;
      // Append: the new token (slot nv - 1) is written here; its key enters
      // the sum from registers. Its rows are read back by the attention only
      // after the block barrier below, which waits for these stores.
      const bool app = a.k_new != nullptr;
      const int slot = app ? nv - 1 : -1;
      typename Quad<KV>::raw knew{};
      if (app) {
        using Raw = typename Quad<KV>::raw;
        const size_t row = (size_t)b * a.hkv + g;
        if (own) {
          knew = Quad<KV>::load((const KV*)a.k_new + row * DK + 4 * dl);
          *(Raw*)(const_cast<KV*>(col) + (size_t)slot * DK) = knew;
        }
        KV* vrow = (KV*)a.vp + (((size_t)pid * a.hkv + g) * P + slot) * a.dv;
        for (int d = 4 * lane; d < a.dv; d += 256)
          *(Raw*)(vrow + d) = Quad<KV>::load((const KV*)a.v_new + row * a.dv + d);
      }
      // Token-order sum; the new token is the page's last, added after the
      // stored ones (the same order as summing it in place).
      const int nsum = app ? nv - 1 : nv;
      float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int t0 = 0; t0 < nsum; t0 += kTok) {
        typename Quad<KV>::raw x[kTok];
#pragma unroll
        for (int t = 0; t < kTok; ++t)
          if (own && t0 + t < nsum) x[t] = Quad<KV>::load(col + (size_t)(t0 + t) * DK);
#pragma unroll
        for (int t = 0; t < kTok; ++t)
          if (own && t0 + t < nsum) {
            const float4 v = Quad<KV>::widen(x[t]);
            s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
          }
      }
      if (app && own) {
        const float4 v = Quad<KV>::widen(knew);
        s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
      }
      const float fn = (float)nv;
      const float4 c4 = make_float4(s4.x / fn, s4.y / fn, s4.z / fn, s4.w / fn);
      if (own) {
        const size_t o = ((size_t)pid * a.hkv + g) * DK + 4 * dl;
        *(float4*)(a.cent + o) = c4;
        if (a.cent_bf16) {
          const uint32_t lo = (uint32_t)f32_to_bf16(c4.x) | ((uint32_t)f32_to_bf16(c4.y) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(c4.z) | ((uint32_t)f32_to_bf16(c4.w) << 16);
          *(uint2*)(a.cent_bf16 + o) = make_uint2(lo, hi);
        }
      }
      // CB16: the page is scored from the copy's value, the bf16 rounding
      const float4 cs =
          CB16 ? make_float4(bf16_to_f32(f32_to_bf16(c4.x)), bf16_to_f32(f32_to_bf16(c4.y)),
                             bf16_to_f32(f32_to_bf16(c4.z)), bf16_to_f32(f32_to_bf16(c4.w)))
               : c4;
      float part = qs.x * cs.x;
      part = fmaf(qs.y, cs.y, part);
      part = fmaf(qs.z, cs.z, part);
      part = fmaf(qs.w, cs.w, part);
      emit(p, part, own);
    }
  }
  __syncthreads();  // every key of the segment is in LDS
  const uint32_t rnd = a.mode == VX_TOPK_APPROX ? a.rnd[seg] : 0u;
  int32_t* const so = sel_global ? a.sel + (size_t)seg * a.stride : nullptr;
  int32_t* const sc = sel_global ? a.sel_count + seg : nullptr;
  if (n > kBlockSelectMin) {
    block_select_keys<NW>(keys, keys + a.cap_keys, keys + a.cap_keys + kSelectHistWords, n, a.k, a.n_sink,
                          a.n_local, a.mode, rnd, so, a.stride, sc, sel_lds, count_lds);
  } else if (w == 0) {
    idle(n, L, true);
    wave_select_keys(keys, n, a.k, a.n_sink, a.n_local, a.mode, rnd, so, a.stride, sc, lane,
                     sel_lds, count_lds);
  } else {
    idle(n, L, false);
  }
}

}  // namespace vx
