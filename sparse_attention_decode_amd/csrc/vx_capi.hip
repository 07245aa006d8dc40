// C ABI of the block top-k sparse-attention decode step: argument checks,
// the workload planner, and kernel dispatch. Every check here runs on the
// host before any HIP call, so a rejected call touches no GPU state.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "vx_internal.h"

namespace {

thread_local std::string g_err;

vx_status fail(vx_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

vx_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return VX_OK;
  return fail(VX_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define VX_CHECK(cond, st, ...) \
  do {                          \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

vx_status check_pages(const vx_pages* p) {
  VX_CHECK(p, VX_ERR_INVALID_ARG, "pages is NULL");
  VX_CHECK(p->batch >= 0, VX_ERR_INVALID_ARG, "batch < 0");
  VX_CHECK(p->page_size == 16 || p->page_size == 64, VX_ERR_UNSUPPORTED,
           "page_size %d (supported: 16, 64)", p->page_size);
  VX_CHECK(p->total_pages >= 0, VX_ERR_INVALID_ARG, "total_pages < 0");
  VX_CHECK(p->max_pages >= 0 && p->max_pages <= p->total_pages, VX_ERR_INVALID_ARG,
           "max_pages %d outside [0, total_pages=%d]", p->max_pages, p->total_pages);
  VX_CHECK(p->total_pages == 0 || p->num_pool_pages >= 1, VX_ERR_INVALID_ARG,
           "num_pool_pages < 1");
  VX_CHECK(p->batch == 0 || (p->indptr && p->seq_lens), VX_ERR_INVALID_ARG,
           "indptr or seq_lens is NULL");
  VX_CHECK(p->total_pages == 0 || p->page_ids, VX_ERR_INVALID_ARG, "page_ids is NULL");
  VX_CHECK(p->batch > 0 || p->total_pages == 0, VX_ERR_INVALID_ARG,
           "total_pages > 0 with batch 0");
  return VX_OK;
}

vx_status check_geom(const vx_geom* g) {
  VX_CHECK(g, VX_ERR_INVALID_ARG, "geom is NULL");
  VX_CHECK(g->num_q_heads >= 1 && g->num_kv_heads >= 1, VX_ERR_INVALID_ARG, "heads < 1");
  VX_CHECK(g->num_q_heads % g->num_kv_heads == 0, VX_ERR_INVALID_ARG,
           "num_q_heads %d not a multiple of num_kv_heads %d", g->num_q_heads, g->num_kv_heads);
  VX_CHECK(g->q_dtype == VX_F32 || g->q_dtype == VX_BF16, VX_ERR_INVALID_ARG, "q_dtype");
  VX_CHECK(g->kv_dtype == VX_F32 || g->kv_dtype == VX_BF16, VX_ERR_INVALID_ARG, "kv_dtype");
  VX_CHECK(g->score_bf16 == 0 || g->score_bf16 == 1, VX_ERR_INVALID_ARG,
           "score_bf16 %d (0 or 1)", g->score_bf16);
  if (g->mla) {
    VX_CHECK(g->num_kv_heads == 1, VX_ERR_INVALID_ARG, "MLA has one latent stream (num_kv_heads 1)");
    VX_CHECK(g->num_q_heads == 16 || g->num_q_heads == 32, VX_ERR_UNSUPPORTED,
             "MLA query heads %d (supported: 16, 32)", g->num_q_heads);
    VX_CHECK(g->head_dim_k == 576 && g->head_dim_v == 512, VX_ERR_UNSUPPORTED,
             "MLA geometry %dx%d (supported: 576 key, 512 value)", g->head_dim_k, g->head_dim_v);
    VX_CHECK(g->q_dtype == VX_BF16 && g->kv_dtype == VX_BF16, VX_ERR_UNSUPPORTED,
             "MLA needs bf16 q and KV");
    VX_CHECK(g->score_dim == 0 || g->score_dim == 576 || g->score_dim == 512, VX_ERR_UNSUPPORTED,
             "MLA score_dim %d (supported: 0 or 576 = all columns, 512 = latent only)",
             g->score_dim);
  } else {
    VX_CHECK(g->head_dim_k == g->head_dim_v, VX_ERR_UNSUPPORTED, "GQA needs head_dim_k == head_dim_v");
    VX_CHECK(g->head_dim_k == 64 || g->head_dim_k == 128, VX_ERR_UNSUPPORTED,
             "head_dim %d (supported: 64, 128)", g->head_dim_k);
    VX_CHECK(g->q_dtype == g->kv_dtype, VX_ERR_UNSUPPORTED, "q and KV dtypes differ");
    VX_CHECK(g->num_kv_heads * g->head_dim_k <= 2048, VX_ERR_UNSUPPORTED,
             "num_kv_heads * head_dim > 2048");
    VX_CHECK(g->score_dim == 0 || g->score_dim == g->head_dim_k, VX_ERR_UNSUPPORTED,
             "GQA scores every column (score_dim 0 or head_dim_k)");
    VX_CHECK(!g->score_bf16 || g->kv_dtype == VX_BF16, VX_ERR_UNSUPPORTED,
             "score_bf16 needs bf16 KV");
  }
  return VX_OK;
}

vx_status check_topk(const vx_pages* p, int32_t k, int32_t n_sink, int32_t n_local, int32_t mode,
                     const uint32_t* rand_u32, const int32_t* sel, int32_t sel_stride,
                     const int32_t* sel_count) {
  VX_CHECK(k >= 0 && n_sink >= 0 && n_local >= 0, VX_ERR_INVALID_ARG,
           "k, n_sink, n_local must be >= 0");
  VX_CHECK((long)k + n_sink + n_local <= sel_stride && sel_stride >= 1, VX_ERR_INVALID_ARG,
           "sel_stride %d < max(1, k + n_sink + n_local)", sel_stride);
  VX_CHECK(mode == VX_TOPK_EXACT || mode == VX_TOPK_APPROX, VX_ERR_INVALID_ARG, "mode %d", mode);
  VX_CHECK(mode != VX_TOPK_APPROX || rand_u32, VX_ERR_INVALID_ARG, "approx mode needs rand_u32");
  VX_CHECK(p->max_pages <= vx::kMaxTopkPages, VX_ERR_UNSUPPORTED,
           "max_pages %d > %d", p->max_pages, vx::kMaxTopkPages);
  VX_CHECK(p->batch == 0 || (sel && sel_count), VX_ERR_INVALID_ARG, "sel or sel_count is NULL");
  return VX_OK;
}

// Waves per block of the stand-alone top-k kernel: as many LDS-resident
// segments as fit 64 KB, at most 4.
int topk_waves(int max_pages) {
  const int cap_keys = (max_pages + 63) / 64 * 64;
  const int wpb = (int)(65536 / ((size_t)cap_keys * 4));
  return wpb < 1 ? 1 : (wpb > 4 ? 4 : wpb);
}

vx_status check_index_args(const vx_pages* pages, const vx_geom* geom, const void* q,
                           const void* k_pool, const float* centroids, const void* cent_bf16,
                           int32_t refresh_newest, float score_scale, const float* scores,
                           int32_t k, int32_t n_sink, int32_t n_local, int32_t mode,
                           const uint32_t* rand_u32, const int32_t* sel, int32_t sel_stride,
                           const int32_t* sel_count) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(refresh_newest == 0 || refresh_newest == 1, VX_ERR_INVALID_ARG,
           "refresh_newest must be 0 or 1");
  VX_CHECK(std::isfinite(score_scale), VX_ERR_INVALID_ARG, "score_scale not finite");
  if ((st = check_topk(pages, k, n_sink, n_local, mode, rand_u32, sel, sel_stride, sel_count)) !=
      VX_OK)
    return st;
  VX_CHECK(pages->batch == 0 || q, VX_ERR_INVALID_ARG, "q is NULL");
  VX_CHECK(pages->total_pages == 0 || scores, VX_ERR_INVALID_ARG, "scores is NULL");
  VX_CHECK(pages->total_pages == 0 || centroids, VX_ERR_INVALID_ARG, "centroids is NULL");
  VX_CHECK(!(geom->mla || geom->score_bf16) || pages->total_pages == 0 || cent_bf16,
           VX_ERR_INVALID_ARG, "%s scores the bf16 centroids: cent_bf16 is NULL",
           geom->mla ? "MLA" : "score_bf16");
  VX_CHECK(!refresh_newest || pages->total_pages == 0 || k_pool, VX_ERR_INVALID_ARG,
           "refresh_newest needs k_pool");
  return VX_OK;
}

// Checks of vx_sparse_decode's own arguments (pages and geometry already
// checked); `launching` adds the pointers a launch needs.
vx_status check_decode_args(const vx_pages* pages, const vx_geom* geom, const void* q,
                            const void* k_pool, const void* v_pool, const int32_t* sel,
                            int32_t sel_stride, const int32_t* sel_count, float sm_scale,
                            const float* out, bool launching) {
  VX_CHECK(sel_stride >= 1, VX_ERR_INVALID_ARG, "sel_stride < 1");
  VX_CHECK(std::isfinite(sm_scale), VX_ERR_INVALID_ARG, "sm_scale not finite");
  if (!geom->mla) {
    const int G = geom->num_q_heads / geom->num_kv_heads;
    VX_CHECK(G == 1 || G == 2 || G == 4 || G == 8, VX_ERR_UNSUPPORTED,
             "GQA group %d (supported: 1, 2, 4, 8)", G);
  } else {
    VX_CHECK(pages->page_size == 64, VX_ERR_UNSUPPORTED, "MLA attention needs page_size 64");
  }
  if (launching) {
    VX_CHECK(pages->batch == 0 || (q && k_pool && sel && sel_count && out), VX_ERR_INVALID_ARG,
             "q, k_pool, sel, sel_count or out is NULL");
    VX_CHECK(geom->mla || pages->batch == 0 || v_pool, VX_ERR_INVALID_ARG, "v_pool is NULL");
  }
  return VX_OK;
}

vx::Meta meta_of(const vx_pages* p) {
  vx::Meta m;
  m.batch = p->batch;
  m.page_size = p->page_size;
  m.pool = p->num_pool_pages;
  m.nnz = p->total_pages;
  m.indptr = p->indptr;
  m.page_ids = p->page_ids;
  m.seq_lens = p->seq_lens;
  return m;
}

int g_cus[64];  // per-device compute-unit count, 0 = not queried yet

vx_status device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev >= 0 && dev < 64 && __atomic_load_n(&g_cus[dev], __ATOMIC_ACQUIRE) > 0) {
    *out = g_cus[dev];
    return VX_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute");
  if (dev >= 0 && dev < 64) __atomic_store_n(&g_cus[dev], n, __ATOMIC_RELEASE);
  *out = n;
  return VX_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kScorePagesPerWave = 8;

// The planner. An attention block serves one (sequence, KV head) for GQA or
// one sequence for MLA, with its waves splitting that selection's chunks;
// when the batch alone gives fewer blocks than compute units, each selection
// is cut into S balanced splits (merged afterwards by log-sum-exp) so that
// about one block runs per compute unit, but no split streams less than
// kMinSplitBytes of keys and values (below that the merge launch costs more
// than the parallelism gains), and no more splits are used than the largest
// split's size needs. No split holds more than kMaxPagesPerSplit pages.
constexpr long kMinSplitBytes = 128 * 1024;

vx_status make_plan(const vx_pages* p, const vx_geom* g, int sel_stride, int num_splits,
                    int num_cus, vx_plan* out) {
  *out = vx_plan{};
  out->num_cus = num_cus;
  const int stride = sel_stride < 1 ? 1 : sel_stride;
  const long items0 = (long)p->batch * (g->mla ? 1 : g->num_kv_heads);
  const int units = stride;  // pages
  const int unit_cap = vx::kMaxPagesPerSplit;
  int S;
  if (num_splits > 0) {
    S = num_splits;
  } else {
    long s = items0 > 0 ? (num_cus + items0 - 1) / items0 : 1;
    const long elt = g->kv_dtype == VX_F32 ? 4 : 2;
    const long row = (g->mla ? g->head_dim_k : g->head_dim_k + g->head_dim_v) * elt;
    const long most = (long)stride * p->page_size * row / kMinSplitBytes;  // a full selection
    if (s > most) s = most;
    S = (int)(s < 1 ? 1 : s);
    if (S > units) S = units;
    // The largest split sets the time; use no more splits than that size
    // needs (fewer partials to write and merge, fewer blocks repeating
    // per-sequence work).
    const int per = (units + S - 1) / S;
    S = (units + per - 1) / per;
  }
  if (S > units) S = units;
  const int min_splits = (units + unit_cap - 1) / unit_cap;
  if (S < min_splits) S = min_splits;
  const int per = (units + S - 1) / S;  // largest split, in units
  out->num_splits = S;
  out->pages_per_split = per;
  out->score_pages_per_block = 4 * kScorePagesPerWave;
  out->score_blocks = (p->total_pages + out->score_pages_per_block - 1) / out->score_pages_per_block;
  out->topk_threads = p->max_pages > vx::kBlockSelectMin ? 512 : 64;
  const int hq = g->num_q_heads, dv = g->head_dim_v;
  size_t ws = 0;
  if (S > 1) {
    ws = align_up((size_t)p->batch * hq * S * dv * sizeof(float), 256);
    ws += align_up((size_t)p->batch * hq * S * 2 * sizeof(float), 256);
  }
  out->workspace_bytes = ws;
  out->fused_step = S == 1 && p->total_pages > 0 &&
                    vx::decode_step_fusable(*g, p->page_size, p->max_pages, sel_stride, false);
  // The whole-step kernel takes one (sequence, KV head) segment per block.
  // When the segments need more than two rounds of blocks over the compute
  // units, the last blocks decide the step's end: order the sequences longest
  // first, so the long segments start early and short ones fill the tail.
  out->order_segments = out->fused_step && items0 > 2L * num_cus &&
                        p->batch <= vx::kMaxOrderedBatch;
  // Up to two rounds of 8-wave blocks are all resident from the start, two
  // per compute unit, and the GPU places block j + num_cus beside block j:
  // a row of long segments and a row of short ones then share each compute
  // unit (ranked inside the step kernel, which is cheaper than a ranking
  // launch for a batch this size).
  const bool bf16_128 = g->kv_dtype == VX_BF16 && g->head_dim_k == 128;
  const int waves = bf16_128 ? vx::gqa_attn_waves(g->num_q_heads / std::max(1, g->num_kv_heads),
                                                  p->max_pages)
                             : 8;
  out->pair_segments = (out->fused_step && waves == 8 && items0 > num_cus &&
                        items0 <= 2L * num_cus && num_cus % g->num_kv_heads == 0 &&
                        p->batch <= vx::kMaxPairedBatch)
                           ? num_cus / g->num_kv_heads
                           : 0;
  return VX_OK;
}

// Workspace of a whole step: vx_sparse_decode's, then (ordered plans) the
// sequence order, 4 bytes per sequence.
size_t step_workspace_bytes(const vx_pages* p, const vx_plan& plan) {
  return plan.workspace_bytes +
         (plan.order_segments ? align_up((size_t)p->batch * sizeof(int32_t), 256) : 0);
}

// Per-split partial outputs and (m, l) pairs in the workspace (S > 1), laid
// out as make_plan sizes them.
void split_buffers(const vx_pages* p, const vx_geom* g, int S, void* ws, float** part_o,
                   float** part_ml) {
  *part_o = nullptr;
  *part_ml = nullptr;
  if (S <= 1) return;
  *part_o = (float*)ws;
  *part_ml = (float*)((char*)ws + align_up((size_t)p->batch * g->num_q_heads * S *
                                               g->head_dim_v * sizeof(float),
                                           256));
}

// Scratch memory of vx_decode_step_static: the split partials of a step,
// in a file-scope device array instead of a caller's workspace. Each device
// that loads the library holds its own copy until the process ends. Host
// code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and kept per device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
void* g_scratch[64];  // per-device address of `scratch`, null until looked up

vx_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  VX_CHECK(dev >= 0 && dev < 64, VX_ERR_UNSUPPORTED, "device %d (supported: 0..63)", dev);
  void* p = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    VX_CHECK(p, VX_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    __atomic_store_n(&g_scratch[dev], p, __ATOMIC_RELEASE);
  }
  *out = p;
  return VX_OK;
}

}  // namespace

extern "C" {

int32_t vx_abi_version(void) { return 8; }

const char* vx_status_string(vx_status s) {
  switch (s) {
    case VX_OK: return "VX_OK";
    case VX_ERR_INVALID_ARG: return "VX_ERR_INVALID_ARG";
    case VX_ERR_UNSUPPORTED: return "VX_ERR_UNSUPPORTED";
    case VX_ERR_WORKSPACE: return "VX_ERR_WORKSPACE";
    case VX_ERR_HIP: return "VX_ERR_HIP";
  }
  return "VX_ERR_UNKNOWN";
}

const char* vx_last_error(void) { return g_err.c_str(); }

vx_status vx_plan_decode(const vx_pages* pages, const vx_geom* geom, int32_t sel_stride,
                         int32_t num_splits, int32_t num_cus, vx_plan* plan) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(plan, VX_ERR_INVALID_ARG, "plan is NULL");
  VX_CHECK(sel_stride >= 1, VX_ERR_INVALID_ARG, "sel_stride < 1");
  if (num_cus <= 0 && (st = device_cus(&num_cus)) != VX_OK) return st;
  return make_plan(pages, geom, sel_stride, num_splits, num_cus, plan);
}

vx_status vx_check_pages(const vx_pages* pages, int32_t* counts, hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  VX_CHECK(counts, VX_ERR_INVALID_ARG, "counts is NULL");
  return hip_status(vx::launch_check_pages(meta_of(pages), pages->max_pages, counts, stream),
                    "page check kernel launch");
}

vx_status vx_centroid_update(const vx_pages* pages, const vx_geom* geom, void* k_pool,
                             void* v_pool, const int32_t* first_token, const void* k_new,
                             const void* v_new, float* centroids, void* cent_bf16,
                             hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(pages->total_pages == 0 || k_pool, VX_ERR_INVALID_ARG, "k_pool is NULL");
  VX_CHECK(centroids, VX_ERR_INVALID_ARG, "centroids is NULL");
  VX_CHECK(!k_new || first_token, VX_ERR_INVALID_ARG, "k_new needs first_token (append mode)");
  VX_CHECK(!v_new || (first_token && v_pool && !geom->mla), VX_ERR_INVALID_ARG,
           "v_new needs first_token and v_pool (and no MLA)");
  VX_CHECK(!(geom->mla && v_pool), VX_ERR_INVALID_ARG, "MLA has no separate v_pool");
  VX_CHECK(geom->mla || !geom->score_bf16 || pages->total_pages == 0 || cent_bf16,
           VX_ERR_INVALID_ARG, "score_bf16 scores the bf16 copy: cent_bf16 is NULL");
  if (pages->batch == 0) return VX_OK;
  const vx::Meta m = meta_of(pages);
  hipError_t e;
  if (!first_token)
    e = vx::launch_centroid_rebuild(m, *geom, k_pool, centroids, (uint16_t*)cent_bf16, stream);
  else
    e = vx::launch_centroid_append(m, *geom, k_pool, v_new ? v_pool : nullptr, first_token,
                                   k_new, v_new, centroids, (uint16_t*)cent_bf16, stream);
  return hip_status(e, "centroid kernel launch");
}

vx_status vx_page_scores(const vx_pages* pages, const vx_geom* geom, const void* q,
                         const void* centroids, float score_scale, float* scores,
                         hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(pages->batch == 0 || q, VX_ERR_INVALID_ARG, "q is NULL");
  VX_CHECK(pages->total_pages == 0 || (centroids && scores), VX_ERR_INVALID_ARG,
           "centroids or scores is NULL");
  VX_CHECK(std::isfinite(score_scale), VX_ERR_INVALID_ARG, "score_scale not finite");
  if (pages->total_pages == 0) return VX_OK;
  const vx::Meta m = meta_of(pages);
  hipError_t e;
  if (geom->mla)
    e = vx::launch_scores_mla_sized(m, *geom, q, nullptr, nullptr,
                                    const_cast<uint16_t*>((const uint16_t*)centroids), 0,
                                    score_scale, scores, pages->max_pages, stream);
  else if (geom->score_bf16)  // centroids is the bf16 copy
    e = vx::launch_scores_gqa(m, *geom, q, nullptr, nullptr,
                              const_cast<uint16_t*>((const uint16_t*)centroids), 0, score_scale,
                              scores, stream);
  else
    e = vx::launch_scores_gqa(m, *geom, q, nullptr, const_cast<float*>((const float*)centroids),
                              nullptr, 0, score_scale, scores, stream);
  return hip_status(e, "score kernel launch");
}

vx_status vx_bounds_update(const vx_pages* pages, const vx_geom* geom, const void* k_pool,
                           const int32_t* first_token, void* bounds, hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(!geom->mla, VX_ERR_UNSUPPORTED, "page bounds are implemented for GQA only");
  VX_CHECK(pages->total_pages == 0 || (k_pool && bounds), VX_ERR_INVALID_ARG,
           "k_pool or bounds is NULL");
  if (pages->batch == 0) return VX_OK;
  return hip_status(vx::launch_bounds_update(meta_of(pages), *geom, k_pool, first_token, bounds,
                                             stream),
                    "bounds kernel launch");
}

vx_status vx_bound_scores(const vx_pages* pages, const vx_geom* geom, const void* q,
                          const void* k_pool, void* bounds, int32_t refresh_newest,
                          float score_scale, float* scores, hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(!geom->mla, VX_ERR_UNSUPPORTED, "page bounds are implemented for GQA only");
  VX_CHECK(refresh_newest == 0 || refresh_newest == 1, VX_ERR_INVALID_ARG,
           "refresh_newest must be 0 or 1");
  VX_CHECK(std::isfinite(score_scale), VX_ERR_INVALID_ARG, "score_scale not finite");
  VX_CHECK(pages->batch == 0 || q, VX_ERR_INVALID_ARG, "q is NULL");
  VX_CHECK(pages->total_pages == 0 || (bounds && scores), VX_ERR_INVALID_ARG,
           "bounds or scores is NULL");
  VX_CHECK(!refresh_newest || pages->total_pages == 0 || k_pool, VX_ERR_INVALID_ARG,
           "refresh_newest needs k_pool");
  if (pages->total_pages == 0) return VX_OK;
  return hip_status(vx::launch_bound_scores(meta_of(pages), *geom, q, k_pool, bounds,
                                            refresh_newest, score_scale, scores,
                                            pages->max_pages, stream),
                    "bound score kernel launch");
}

vx_status vx_topk_pages(const vx_pages* pages, int32_t num_kv_heads, const float* scores,
                        int32_t k, int32_t n_sink, int32_t n_local, int32_t mode,
                        const uint32_t* rand_u32, int32_t* sel, int32_t sel_stride,
                        int32_t* sel_count, hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  VX_CHECK(num_kv_heads >= 1, VX_ERR_INVALID_ARG, "num_kv_heads < 1");
  if ((st = check_topk(pages, k, n_sink, n_local, mode, rand_u32, sel, sel_stride, sel_count)) !=
      VX_OK)
    return st;
  VX_CHECK(pages->total_pages == 0 || scores, VX_ERR_INVALID_ARG, "scores is NULL");
  if (pages->batch == 0) return VX_OK;
  const vx::Meta m = meta_of(pages);
  hipError_t e = vx::launch_topk_sized(m, num_kv_heads, scores, k, n_sink, n_local, mode, rand_u32,
                                       sel, sel_stride, sel_count, pages->max_pages,
                                       topk_waves(pages->max_pages), stream);
  return hip_status(e, "top-k kernel launch");
}

vx_status vx_index_pages(const vx_pages* pages, const vx_geom* geom, const void* q,
                         const void* k_pool, float* centroids, void* cent_bf16,
                         int32_t refresh_newest, float score_scale, float* scores, int32_t k,
                         int32_t n_sink, int32_t n_local, int32_t mode, const uint32_t* rand_u32,
                         int32_t* sel, int32_t sel_stride, int32_t* sel_count,
                         hipStream_t stream) {
  vx_status st;
  if ((st = check_index_args(pages, geom, q, k_pool, centroids, cent_bf16, refresh_newest,
                             score_scale, scores, k, n_sink, n_local, mode, rand_u32, sel,
                             sel_stride, sel_count)) != VX_OK)
    return st;
  if (pages->batch == 0) return VX_OK;
  const vx::Meta m = meta_of(pages);
  hipError_t e = hipSuccess;
  if (pages->total_pages > 0) {
    if (geom->mla) {
      e = vx::launch_scores_mla_sized(m, *geom, q, k_pool, centroids, (uint16_t*)cent_bf16,
                                      refresh_newest, score_scale, scores, pages->max_pages,
                                      stream);
    } else {
      e = vx::launch_index_gqa(m, *geom, q, k_pool, centroids, (uint16_t*)cent_bf16,
                               refresh_newest, score_scale, scores, k, n_sink, n_local, mode,
                               rand_u32, sel, sel_stride, sel_count, pages->max_pages, stream);
      return hip_status(e, "indexer kernel launch");
    }
    if (e != hipSuccess) return hip_status(e, "score kernel launch");
  }
  e = vx::launch_topk_sized(m, geom->num_kv_heads, scores, k, n_sink, n_local, mode, rand_u32, sel,
                            sel_stride, sel_count, pages->max_pages, topk_waves(pages->max_pages),
                            stream);
  return hip_status(e, "top-k kernel launch");
}

vx_status vx_sparse_decode(const vx_pages* pages, const vx_geom* geom, const void* q,
                           const void* k_pool, const void* v_pool, const int32_t* sel,
                           int32_t sel_stride, const int32_t* sel_count, float sm_scale,
                           float* out, float* lse, int32_t num_splits, void* workspace,
                           size_t* workspace_bytes, hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(workspace_bytes, VX_ERR_INVALID_ARG, "workspace_bytes is NULL");
  if ((st = check_decode_args(pages, geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                              out, workspace != nullptr)) != VX_OK)
    return st;
  int cus = 0;
  if ((st = device_cus(&cus)) != VX_OK) return st;
  vx_plan plan;
  if ((st = make_plan(pages, geom, sel_stride, num_splits, cus, &plan)) != VX_OK) return st;
  if (!workspace) {
    *workspace_bytes = plan.workspace_bytes;
    return VX_OK;
  }
  VX_CHECK(*workspace_bytes >= plan.workspace_bytes, VX_ERR_WORKSPACE,
           "workspace %zu bytes < %zu needed", *workspace_bytes, plan.workspace_bytes);
  VX_CHECK(pages->batch == 0 || q, VX_ERR_INVALID_ARG, "q is NULL");
  if (pages->batch == 0) return VX_OK;
  const vx::Meta m = meta_of(pages);
  const int S = plan.num_splits;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  split_buffers(pages, geom, S, workspace, &part_o, &part_ml);
  hipError_t e;
  if (geom->mla)
    e = vx::launch_attention_mla(m, *geom, q, k_pool, sel, sel_stride, sel_count, sm_scale, S,
                                 plan.pages_per_split, out, lse, part_o, part_ml, stream);
  else
    e = vx::launch_attention_gqa(m, *geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                                 S, plan.pages_per_split, out, lse, part_o, part_ml,
                                 pages->max_pages, stream);
  if (e != hipSuccess) return hip_status(e, "attention kernel launch");
  if (S > 1) {
    e = vx::launch_merge(pages->batch, geom->num_q_heads, geom->head_dim_v, S, part_o, part_ml, out,
                         lse, stream);
    if (e != hipSuccess) return hip_status(e, "merge kernel launch");
  }
  return VX_OK;
}

namespace {

// vx_decode_step, and with k_new (append) vx_append_decode_step: the new
// token's rows are written and the newest page's centroid recomputed, by the
// whole-step kernel's refresh when the step is one kernel, else by the
// append kernel before the step's kernels (which then skip the refresh).
vx_status decode_step_impl(const vx_pages* pages, const vx_geom* geom, const void* q,
                           const void* k_pool, const void* v_pool, const void* k_new,
                           const void* v_new, float* centroids, void* cent_bf16,
                           int32_t refresh_newest, float score_scale, float sm_scale, int32_t k,
                           int32_t n_sink, int32_t n_local, int32_t mode,
                           const uint32_t* rand_u32, float* scores, int32_t* sel,
                           int32_t sel_stride, int32_t* sel_count, float* out, float* lse,
                           int32_t num_splits, void* workspace, size_t* workspace_bytes,
                           hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(workspace_bytes, VX_ERR_INVALID_ARG, "workspace_bytes is NULL");
  if (k_new || v_new) {
    VX_CHECK(pages->batch == 0 || k_new, VX_ERR_INVALID_ARG, "k_new is NULL");
    VX_CHECK(geom->mla ? !v_new : (pages->batch == 0 || v_new), VX_ERR_INVALID_ARG,
             geom->mla ? "MLA takes no v_new (values are the latent rows)" : "v_new is NULL");
  }
  if ((st = check_decode_args(pages, geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                              out, workspace != nullptr)) != VX_OK)
    return st;
  if (workspace &&
      (st = check_index_args(pages, geom, q, k_pool, centroids, cent_bf16,
                             k_new ? 1 : refresh_newest, score_scale, scores, k, n_sink, n_local,
                             mode, rand_u32, sel, sel_stride, sel_count)) != VX_OK)
    return st;
  int cus = 0;
  if ((st = device_cus(&cus)) != VX_OK) return st;
  vx_plan plan;
  if ((st = make_plan(pages, geom, sel_stride, num_splits, cus, &plan)) != VX_OK) return st;
  const size_t need = step_workspace_bytes(pages, plan);
  if (!workspace) {
    *workspace_bytes = need;
    return VX_OK;
  }
  VX_CHECK(*workspace_bytes >= need, VX_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
           *workspace_bytes, need);
  if (pages->batch == 0) return VX_OK;
  if (plan.num_splits == 1 && pages->total_pages > 0 &&
      vx::decode_step_fusable(*geom, pages->page_size, pages->max_pages, sel_stride, false)) {
    int32_t* order = nullptr;
    hipError_t e = hipSuccess;
    if (plan.order_segments) {
      order = (int32_t*)((char*)workspace + plan.workspace_bytes);
      e = vx::launch_rank_sequences(meta_of(pages), order, stream);
      if (e != hipSuccess) return hip_status(e, "sequence order kernel launch");
    }
    e = vx::launch_decode_step_gqa(
        meta_of(pages), *geom, q, k_pool, v_pool, centroids, (uint16_t*)cent_bf16, nullptr,
        k_new ? 1 : refresh_newest, score_scale, sm_scale, scores, k, n_sink, n_local, mode,
        rand_u32, sel, sel_stride, sel_count, out, lse, pages->max_pages, order,
        plan.pair_segments, k_new, v_new, stream);
    return hip_status(e, "decode step kernel launch");
  }
  if (k_new && pages->total_pages > 0) {
    hipError_t e = vx::launch_centroid_append(meta_of(pages), *geom, const_cast<void*>(k_pool),
                                              const_cast<void*>(v_new ? v_pool : nullptr), nullptr,
                                              k_new, v_new, centroids, (uint16_t*)cent_bf16,
                                              stream);
    if (e != hipSuccess) return hip_status(e, "centroid kernel launch");
  }
  if (geom->mla && pages->total_pages > 0 &&
      vx::decode_step_mla_fusable(pages->max_pages, sel_stride)) {
    // scores, then selection + attention in one kernel, then the merge (a
    // merge by the last split block to finish was measured slower: that block
    // reads every split's partials alone)
    const vx::Meta m = meta_of(pages);
    const int S = plan.num_splits;
    float* part_o = nullptr;
    float* part_ml = nullptr;
    split_buffers(pages, geom, S, workspace, &part_o, &part_ml);
    // With the newest page forced (n_local >= 1) its score takes no part in
    // the selections, so its refresh runs in extra blocks of the step kernel,
    // beside the attention, instead of at the end of the scorer; the scorer
    // scores it from the old centroid and the refresh then writes its score.
    const int late = refresh_newest && n_local >= 1;
    hipError_t e = vx::launch_scores_mla_sized(m, *geom, q, k_pool, centroids,
                                               (uint16_t*)cent_bf16, late ? 0 : refresh_newest,
                                               score_scale, scores, pages->max_pages, stream);
    if (e != hipSuccess) return hip_status(e, "score kernel launch");
    e = vx::launch_decode_step_mla(m, *geom, q, k_pool, scores, k, n_sink, n_local, mode,
                                   rand_u32, sel, sel_stride, sel_count, sm_scale, S, out, lse,
                                   part_o, part_ml, pages->max_pages, late, centroids,
                                   (uint16_t*)cent_bf16, score_scale, stream);
    if (e != hipSuccess) return hip_status(e, "decode step kernel launch");
    if (S > 1) {
      e = vx::launch_merge(pages->batch, geom->num_q_heads, geom->head_dim_v, S, part_o, part_ml,
                           out, lse, stream);
      if (e != hipSuccess) return hip_status(e, "merge kernel launch");
    }
    return VX_OK;
  }
  if ((st = vx_index_pages(pages, geom, q, k_pool, centroids, cent_bf16, refresh_newest,
                           score_scale, scores, k, n_sink, n_local, mode, rand_u32, sel,
                           sel_stride, sel_count, stream)) != VX_OK)
    return st;
  return vx_sparse_decode(pages, geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                          out, lse, num_splits, workspace, workspace_bytes, stream);
}

}  // namespace

vx_status vx_decode_step(const vx_pages* pages, const vx_geom* geom, const void* q,
                         const void* k_pool, const void* v_pool, float* centroids,
                         void* cent_bf16, int32_t refresh_newest, float score_scale,
                         float sm_scale, int32_t k, int32_t n_sink, int32_t n_local, int32_t mode,
                         const uint32_t* rand_u32, float* scores, int32_t* sel,
                         int32_t sel_stride, int32_t* sel_count, float* out, float* lse,
                         int32_t num_splits, void* workspace, size_t* workspace_bytes,
                         hipStream_t stream) {
  return decode_step_impl(pages, geom, q, k_pool, v_pool, nullptr, nullptr, centroids, cent_bf16,
                          refresh_newest, score_scale, sm_scale, k, n_sink, n_local, mode,
                          rand_u32, scores, sel, sel_stride, sel_count, out, lse, num_splits,
                          workspace, workspace_bytes, stream);
}

vx_status vx_append_decode_step(const vx_pages* pages, const vx_geom* geom, const void* q,
                                void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                float* centroids, void* cent_bf16, float score_scale,
                                float sm_scale, int32_t k, int32_t n_sink, int32_t n_local,
                                int32_t mode, const uint32_t* rand_u32, float* scores,
                                int32_t* sel, int32_t sel_stride, int32_t* sel_count, float* out,
                                float* lse, int32_t num_splits, void* workspace,
                                size_t* workspace_bytes, hipStream_t stream) {
  // batch > 0 needs k_new (and v_new unless MLA); checked in decode_step_impl,
  // which this call reaches with k_new set whenever there are sequences.
  VX_CHECK(k_new || !pages || pages->batch == 0, VX_ERR_INVALID_ARG, "k_new is NULL");
  return decode_step_impl(pages, geom, q, k_pool, v_pool, k_new, v_new, centroids, cent_bf16, 0,
                          score_scale, sm_scale, k, n_sink, n_local, mode, rand_u32, scores, sel,
                          sel_stride, sel_count, out, lse, num_splits, workspace, workspace_bytes,
                          stream);
}

vx_status vx_decode_step_static(const vx_pages* pages, const vx_geom* geom, const void* q,
                                const void* k_pool, const void* v_pool, float* centroids,
                                void* cent_bf16, int32_t refresh_newest, float score_scale,
                                float sm_scale, int32_t k, int32_t n_sink, int32_t n_local,
                                int32_t mode, const uint32_t* rand_u32, float* scores,
                                int32_t* sel, int32_t sel_stride, int32_t* sel_count, float* out,
                                float* lse, int32_t num_splits, hipStream_t stream) {
  vx_status st;
  // Every argument check of a launching vx_decode_step, before any HIP call.
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  if ((st = check_decode_args(pages, geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                              out, true)) != VX_OK)
    return st;
  if ((st = check_index_args(pages, geom, q, k_pool, centroids, cent_bf16, refresh_newest,
                             score_scale, scores, k, n_sink, n_local, mode, rand_u32, sel,
                             sel_stride, sel_count)) != VX_OK)
    return st;
  size_t need = 0;
  // Size query of the same call (host only, no launch), then the limit.
  if ((st = vx_decode_step(pages, geom, q, k_pool, v_pool, centroids, cent_bf16, refresh_newest,
                           score_scale, sm_scale, k, n_sink, n_local, mode, rand_u32, scores,
                           sel, sel_stride, sel_count, out, lse, num_splits, nullptr, &need,
                           stream)) != VX_OK)
    return st;
  VX_CHECK(need <= kStaticScratchBytes, VX_ERR_WORKSPACE,
           "this step needs %zu bytes of scratch; the static scratch holds %zu (fewer splits or "
           "a smaller batch fit, or call vx_decode_step with a workspace)",
           need, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != VX_OK) return st;
  size_t have = kStaticScratchBytes;
  return vx_decode_step(pages, geom, q, k_pool, v_pool, centroids, cent_bf16, refresh_newest,
                        score_scale, sm_scale, k, n_sink, n_local, mode, rand_u32, scores, sel,
                        sel_stride, sel_count, out, lse, num_splits, ws, &have, stream);
}

vx_status vx_bound_decode_step(const vx_pages* pages, const vx_geom* geom, const void* q,
                               const void* k_pool, const void* v_pool, void* bounds,
                               int32_t refresh_newest, float score_scale, float sm_scale,
                               int32_t k, int32_t n_sink, int32_t n_local, int32_t mode,
                               const uint32_t* rand_u32, float* scores, int32_t* sel,
                               int32_t sel_stride, int32_t* sel_count, float* out, float* lse,
                               int32_t num_splits, void* workspace, size_t* workspace_bytes,
                               hipStream_t stream) {
  vx_status st;
  if ((st = check_pages(pages)) != VX_OK) return st;
  if ((st = check_geom(geom)) != VX_OK) return st;
  VX_CHECK(!geom->mla, VX_ERR_UNSUPPORTED, "page bounds are implemented for GQA only");
  VX_CHECK(workspace_bytes, VX_ERR_INVALID_ARG, "workspace_bytes is NULL");
  if ((st = check_decode_args(pages, geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                              out, workspace != nullptr)) != VX_OK)
    return st;
  if (workspace) {
    VX_CHECK(refresh_newest == 0 || refresh_newest == 1, VX_ERR_INVALID_ARG,
             "refresh_newest must be 0 or 1");
    VX_CHECK(std::isfinite(score_scale), VX_ERR_INVALID_ARG, "score_scale not finite");
    if ((st = check_topk(pages, k, n_sink, n_local, mode, rand_u32, sel, sel_stride,
                         sel_count)) != VX_OK)
      return st;
    VX_CHECK(pages->total_pages == 0 || (bounds && scores), VX_ERR_INVALID_ARG,
             "bounds or scores is NULL");
  }
  int cus = 0;
  if ((st = device_cus(&cus)) != VX_OK) return st;
  vx_plan plan;
  if ((st = make_plan(pages, geom, sel_stride, num_splits, cus, &plan)) != VX_OK) return st;
  const bool fused = plan.num_splits == 1 && pages->total_pages > 0 &&
                     vx::decode_step_fusable(*geom, pages->page_size, pages->max_pages,
                                             sel_stride, true);
  plan.order_segments = plan.order_segments && fused;
  const size_t need = step_workspace_bytes(pages, plan);
  if (!workspace) {
    *workspace_bytes = need;
    return VX_OK;
  }
  VX_CHECK(*workspace_bytes >= need, VX_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
           *workspace_bytes, need);
  if (pages->batch == 0) return VX_OK;
  if (fused) {
    int32_t* order = nullptr;
    hipError_t e = hipSuccess;
    if (plan.order_segments) {
      order = (int32_t*)((char*)workspace + plan.workspace_bytes);
      e = vx::launch_rank_sequences(meta_of(pages), order, stream);
      if (e != hipSuccess) return hip_status(e, "sequence order kernel launch");
    }
    e = vx::launch_decode_step_gqa(
        meta_of(pages), *geom, q, k_pool, v_pool, nullptr, nullptr, bounds, refresh_newest,
        score_scale, sm_scale, scores, k, n_sink, n_local, mode, rand_u32, sel, sel_stride,
        sel_count, out, lse, pages->max_pages, order, plan.pair_segments, nullptr, nullptr,
        stream);
    return hip_status(e, "decode step kernel launch");
  }
  if ((st = vx_bound_scores(pages, geom, q, k_pool, bounds, refresh_newest, score_scale, scores,
                            stream)) != VX_OK)
    return st;
  if ((st = vx_topk_pages(pages, geom->num_kv_heads, scores, k, n_sink, n_local, mode, rand_u32,
                          sel, sel_stride, sel_count, stream)) != VX_OK)
    return st;
  return vx_sparse_decode(pages, geom, q, k_pool, v_pool, sel, sel_stride, sel_count, sm_scale,
                          out, lse, num_splits, workspace, workspace_bytes, stream);
}

}  // extern "C"
