/*
 * vx.h -- C ABI of the block top-k sparse-attention decode step (gfx950).
 *
 * The step is the block top-k method of the Vortex paper note
 * ("Vortex: Efficient and Programmable Sparse Attention Serving for AI
 * Agents", papers.chlience.com), section "System design > 1. vFlow":
 *   cache stage    per-page key centroid, query independent  -> vx_centroid_update
 *   indexer        query x centroid scores                    -> vx_page_scores
 *                  top-k pages per (sequence, KV head)        -> vx_topk_pages
 *                  both, fused with the newest-page refresh   -> vx_index_pages
 *   page table     device-side check of its contract         -> vx_check_pages
 *   whole step     indexer + attention, fused where possible  -> vx_decode_step
 *                  the same, without a workspace argument     -> vx_decode_step_static
 *   attention      exact softmax over the selected pages      -> vx_sparse_decode
 * Section "System design > 2. vTensor" gives the paged layout (a tensor with
 * batch size, a pointer array and a page-index structure): vx_pages below.
 * Section "System design > 3. Execution backend" gives the workload planner
 * (vx_plan_decode) and the radix top-k with its approximate mode.
 * The Quest-style indexer the paper note measures against ("Paper context",
 * "Key results > User-side latency") is an alternative cache stage and
 * scorer: page bounds -> vx_bounds_update, bound scores -> vx_bound_scores;
 * its selection and attention are vx_topk_pages and vx_sparse_decode, and
 * vx_bound_decode_step runs the whole step (one kernel where it fits).
 *
 * Conventions shared by every entry point
 *   - Every buffer argument is DEVICE memory owned by the caller, unless the
 *     comment says "host". The library allocates nothing and keeps no
 *     pointer after a call returns.
 *   - Calls are asynchronous and ordered on `stream`; none synchronises the
 *     host. A call returns once its kernels are enqueued.
 *   - Arguments are validated on the host before any GPU work. A bad
 *     argument returns VX_ERR_INVALID_ARG, an unsupported shape or dtype
 *     VX_ERR_UNSUPPORTED, a short workspace VX_ERR_WORKSPACE; nothing is
 *     launched then. A failed launch returns VX_ERR_HIP. vx_last_error()
 *     returns a thread-local message for the last failure.
 *   - Device-side contract (not checked on the host, which never reads device
 *     memory): 0 <= seq_lens[b] <= (indptr[b+1]-indptr[b]) * page_size and
 *     0 <= page_ids[j] < num_pool_pages. A sequence with seq_lens[b] = 0 is
 *     an idle slot: no page scored, an empty selection, out = 0 and
 *     lse = -inf. Kernels clamp both so that no access leaves its buffer;
 *     results for a sequence that breaks them are unspecified.
 *   - Entry points are reentrant; the only library state is per device: a
 *     cache of the compute-unit count, and the address of the scratch array
 *     of vx_decode_step_static (a device array in the library's code object,
 *     loaded with it; no entry point allocates).
 *
 * Memory layouts (row-major, innermost last)
 *   q          [B][Hq][Dk]                     q_dtype
 *   k_pool     [num_pool_pages][Hkv][P][Dk]    kv_dtype
 *   v_pool     [num_pool_pages][Hkv][P][Dv]    kv_dtype  (MLA: unused, V = K[..., :Dv])
 *   centroids  [num_pool_pages][Hkv][Dk]       fp32      (indexed by physical page)
 *   cent_bf16  [num_pool_pages][Hkv][Dk]       bf16      (RNE of the fp32 centroid)
 *   bounds     [num_pool_pages][Hkv][Dk/4][2][4] kv_dtype (per 4 dims: 4 key minima, 4 maxima)
 *   scores     [Hkv][total_pages]              fp32      (entry j of page table)
 *   sel        [B][Hkv][sel_stride]            int32     logical page ids, ascending, -1 padded
 *   sel_count  [B][Hkv]                        int32
 *   out        [B][Hq][Dv]                     fp32
 *   lse        [B][Hq]                         fp32      natural log
 * Query head h reads KV head h / (Hq / Hkv).
 */
#ifndef VX_H_
#define VX_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vx_status {
  VX_OK = 0,
  VX_ERR_INVALID_ARG = 1,
  VX_ERR_UNSUPPORTED = 2,
  VX_ERR_WORKSPACE = 3,
  VX_ERR_HIP = 4
} vx_status;

typedef enum vx_dtype { VX_F32 = 0, VX_BF16 = 1 } vx_dtype;

typedef enum vx_topk_mode {
  VX_TOPK_EXACT = 0,  /* radix select, exact ranking */
  VX_TOPK_APPROX = 1  /* remap + one digit pass + stochastic boundary fill */
} vx_topk_mode;

/* Paged, ragged batch metadata (the page-index structure of a vTensor).
 * Device arrays: indptr[B+1] (indptr[0] = 0, non-decreasing), page_ids
 * [total_pages] physical page of each page-table entry, seq_lens[B] valid
 * tokens. Sequence b owns entries indptr[b] .. indptr[b+1]-1; its logical
 * page p (p < ceil(seq_lens[b] / page_size)) is physical page
 * page_ids[indptr[b] + p]. Entries past the pages in use are capacity for
 * appended tokens. Host ints total_pages (= indptr[B]) and max_pages
 * (= max_b indptr[b+1]-indptr[b]) size the launches without a device read. */
typedef struct vx_pages {
  int32_t batch;
  int32_t page_size;      /* 16 or 64 */
  int32_t num_pool_pages;
  int32_t total_pages;    /* host copy of indptr[B] */
  int32_t max_pages;      /* host copy of the largest per-sequence capacity */
  const int32_t* indptr;
  const int32_t* page_ids;
  const int32_t* seq_lens;
} vx_pages;

/* Head geometry. GQA: Hkv KV heads, Dk == Dv in {64, 128}. MLA (mla = 1):
 * one latent stream (Hkv = 1), Dk = 576 (512 latent + 64 rope), Dv = 512,
 * values are the first Dv columns of the key rows. */
typedef struct vx_geom {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim_k;
  int32_t head_dim_v;
  int32_t mla;
  vx_dtype q_dtype;
  vx_dtype kv_dtype;
  /* Columns the indexer scores: 0 or head_dim_k = all of them. MLA also
   * takes 512: the latent columns only, a rope-unaware indexer (Vortex paper
   * note, "Key results > MLA": routing on the rope part matters; this option
   * measures how much). Attention always uses every column. */
  int32_t score_dim;
  /* GQA with bf16 KV: 1 scores the pages on cent_bf16, the round-to-nearest-
   * even bf16 copy of the fp32 centroids, instead of the fp32 rows (the
   * indexer then reads half the bytes); every call that scores then needs
   * cent_bf16 (vx_page_scores takes the copy as its `centroids`), and so
   * does vx_centroid_update, which keeps the copy. The
   * pages leave the centroids' storage precision open; the scores are the
   * fp32 dot of the group-summed query with the bf16 values. 0: the fp32
   * rows. Any other value: VX_ERR_INVALID_ARG; 1 with fp32 KV:
   * VX_ERR_UNSUPPORTED. MLA always scores the bf16 copy and ignores it, and
   * so do the Quest-style entry points (vx_bound_*), which score bounds. */
  int32_t score_bf16;
} vx_geom;

/* Launch plan chosen by the workload planner (host only). */
typedef struct vx_plan {
  int32_t num_splits;        /* attention work items per (sequence, KV head) */
  int32_t pages_per_split;   /* selected pages each split streams */
  int32_t score_pages_per_block;
  int32_t score_blocks;
  int32_t topk_threads;      /* threads per (sequence, KV head) segment */
  int32_t num_cus;
  int32_t fused_step;        /* 1: vx_decode_step runs as one kernel */
  size_t workspace_bytes;    /* what vx_sparse_decode needs for this plan */
  int32_t order_segments;    /* 1: vx_decode_step orders the sequences longest
                                first on the device (segments span more than
                                two rounds of blocks); its workspace then
                                holds 4 more bytes per sequence */
  int32_t pair_segments;     /* R > 0: every whole-step block is resident
                                from the start, two per compute unit, and
                                block rows i and i + R (Hkv blocks a row)
                                share compute units: the step kernel ranks
                                the sequences by pages in use itself and
                                gives rows i < R the longest, row R + k the
                                k-th shortest; 0: not paired */
} vx_plan;

/* Cache stage: refresh the key centroids of pages.
 * (Vortex paper note, "System design > 1. vFlow": the cache stage precomputes
 * a query-independent statistic per block; for block top-k the key centroid.)
 *
 * centroid[pid][g][:] = (sum over the page's valid tokens t, in token order,
 * of K[pid][g][t][:] in fp32) / n_valid, one IEEE fp32 divide;
 * cent_bf16 (nullable) receives its round-to-nearest-even bf16 copy.
 * Pages past a sequence's last token get zeros.
 *
 * first_token == NULL: rebuild every page-table entry (setup / resume).
 * first_token != NULL ([B] device): refresh, for each sequence b, the pages
 *   holding tokens first_token[b] .. seq_lens[b]-1. A negative value counts
 *   from the end (seq_lens[b] + first_token[b]), so a constant -1 refreshes
 *   only the newest token's page at every decode step. Each refreshed page is
 *   recomputed from its tokens, so the result equals a rebuild bit for bit.
 * k_new / v_new (nullable, require first_token): [B][Hkv][Dk] and
 *   [B][Hkv][Dv] in kv_dtype; written first into the slot of token
 *   seq_lens[b]-1 of k_pool / v_pool (v_new needs v_pool, and is ignored for
 *   MLA). k_pool is only written when k_new is given. */
vx_status vx_centroid_update(const vx_pages* pages, const vx_geom* geom,
                             void* k_pool, void* v_pool,
                             const int32_t* first_token,
                             const void* k_new, const void* v_new,
                             float* centroids, void* cent_bf16,
                             hipStream_t stream);

/* Indexer scoring (Vortex paper note, "System design > 1. vFlow": a matrix
 * product of the query with the centroids).
 * GQA: scores[g][j] = score_scale * sum_{h in group g} q[b][h] . centroids[pid][g]
 *   with fp32 centroids, evaluated as the dot of the fp32 group-summed query
 *   with the centroid row; with geom->score_bf16, centroids is the bf16 copy
 *   [pool][Hkv][Dk] and the same dot runs on its values.
 * MLA: centroids is the bf16 copy [pool][576]; the [Hq x 576] x [576 x pages]
 *   product runs on bf16 MFMA with fp32 accumulation and is summed over the
 *   query heads: scores[0][j] = score_scale * sum_h q[b][h] . cent_bf16[pid].
 * j runs over the entries of sequence b that are in use (p < ceil(L/P));
 * other entries of `scores` are left untouched. */
vx_status vx_page_scores(const vx_pages* pages, const vx_geom* geom,
                         const void* q, const void* centroids,
                         float score_scale, float* scores, hipStream_t stream);

/* Indexer selection: per (sequence b, KV head g), keep the forced pages (the
 * first n_sink pages and the last n_local pages) plus the top-k other pages
 * ranked by (score descending, logical page index ascending); -0.0 and +0.0
 * rank equal. (Vortex paper note, "System design > 1. vFlow": keep the top-k
 * blocks; "System design > 3. Execution backend": radix top-k, with
 * stochastic early termination and remapping as an approximate option.)
 * sel[b][g][0..sel_count[b][g]) = chosen logical ids ascending, -1 after.
 * sel_stride >= k + n_sink + n_local. Scores must be finite.
 * mode VX_TOPK_APPROX: candidates' scores are mapped affinely onto 256
 *   buckets (fp32: w = max-min, bucket = min(255, floor((s-min)*(256/w))));
 *   one histogram pass finds the boundary bucket; every candidate above it is
 *   kept and the remaining r places go to r members of the boundary bucket
 *   taken cyclically in index order from offset rand_u32[b*Hkv+g] mod
 *   (members). rand_u32 ([B][Hkv] device) is required in this mode only. */
vx_status vx_topk_pages(const vx_pages* pages, int32_t num_kv_heads,
                        const float* scores, int32_t k, int32_t n_sink,
                        int32_t n_local, int32_t mode, const uint32_t* rand_u32,
                        int32_t* sel, int32_t sel_stride, int32_t* sel_count,
                        hipStream_t stream);

/* Quest-style cache stage (GQA only; MLA returns VX_ERR_UNSUPPORTED). The
 * mechanism is Quest's (Tang et al., "Quest: Query-Aware Sparsity for
 * Efficient Long-Context LLM Inference", ICML 2024), the other baseline of
 * the Vortex paper note ("Paper context", "Key results > User-side
 * latency"): per page and KV head, the elementwise minimum and maximum of
 * the keys of its valid tokens.
 * bounds[pid][g][d/4][0][d%4] = min over valid t of K[pid][g][t][d],
 * bounds[pid][g][d/4][1][d%4] = max over the same tokens, in kv_dtype (exact:
 * the extremes of bf16 keys are bf16 values; the interleaving gives a 16-byte
 * load both bounds of 4 dims). Pages past a sequence's last token get zeros.
 * first_token == NULL: rebuild every page-table entry. Otherwise ([B]
 * device) refresh each sequence's pages holding tokens first_token[b] ..
 * seq_lens[b]-1, a negative value counting from the end (-1: the newest
 * token's page). Each refreshed page is recomputed from its keys, so the
 * result equals a rebuild bit for bit. k_pool is only read: the caller
 * writes appended keys into it first. */
vx_status vx_bounds_update(const vx_pages* pages, const vx_geom* geom,
                           const void* k_pool, const int32_t* first_token,
                           void* bounds, hipStream_t stream);

/* Quest-style scores (GQA only): with Q[g] = sum over the query heads h of
 * group g of q[b][h] (fp32, head order) times score_scale,
 *   scores[g][j] = sum_d max(Q[g][d] * lo[d], Q[g][d] * hi[d]),
 * lo / hi the bounds rows of entry j's page: an upper bound of
 * score_scale * sum_h q[b][h] . K_t over every valid token t of the page
 * (the least one that depends on the bounds alone).
 * refresh_newest = 1 first recomputes, from k_pool, the bounds of the page
 * holding each sequence's newest token (exactly vx_bounds_update with
 * first_token[b] = -1) and scores that page from them; no physical page that
 * is some sequence's newest page may then appear in another sequence's page
 * table. j runs over the entries in use; other entries of `scores` are left
 * untouched. The scores feed vx_topk_pages. */
vx_status vx_bound_scores(const vx_pages* pages, const vx_geom* geom,
                          const void* q, const void* k_pool, void* bounds,
                          int32_t refresh_newest, float score_scale,
                          float* scores, hipStream_t stream);

/* Indexer, fused (Vortex paper note, "System design > 3. Execution backend":
 * sequence-local operators are fused). One call runs
 *   1. refresh_newest = 1: the cache-stage refresh of the page holding each
 *      sequence's newest token (exactly vx_centroid_update with
 *      first_token[b] = -1 and no k_new: centroids, and cent_bf16 when given,
 *      are rewritten for that page);
 *   2. the scores of vx_page_scores (GQA reads `centroids`, or `cent_bf16`
 *      with geom->score_bf16; MLA `cent_bf16`);
 *   3. the selection of vx_topk_pages over those scores;
 * and writes the same bits as those three calls in that order. For GQA it
 * is one kernel with a block per (sequence, KV head): the block streams that
 * head's slice of the sequence's centroid rows, keeps the scores as keys in
 * LDS and selects from them, so no block waits for another. MLA runs the
 * three steps as consecutive kernels.
 * With refresh_newest = 1, no physical page that is some sequence's newest
 * page may appear in another sequence's page table in the same call. */
vx_status vx_index_pages(const vx_pages* pages, const vx_geom* geom,
                         const void* q, const void* k_pool,
                         float* centroids, void* cent_bf16,
                         int32_t refresh_newest, float score_scale,
                         float* scores, int32_t k, int32_t n_sink,
                         int32_t n_local, int32_t mode,
                         const uint32_t* rand_u32, int32_t* sel,
                         int32_t sel_stride, int32_t* sel_count,
                         hipStream_t stream);

/* Sparse attention (Vortex paper note, "System design > 1. vFlow": exact
 * softmax attention on the selected blocks). For query head h of sequence b
 * (KV head g = h / G) over the valid tokens t of the pages in
 * sel[b][g][0..sel_count[b][g]):
 *   z_t = sm_scale * q[b][h] . K_t,  out[b][h] = sum_t softmax(z)_t V_t,
 *   lse[b][h] = ln sum_t exp(z_t) (nullable).
 * Split-K: the planner (or num_splits > 0) cuts each selection into splits
 * processed in parallel; their partial results are merged by log-sum-exp.
 * A (b, h) with an empty selection gets out = 0, lse = -inf.
 * workspace == NULL: only writes the bytes needed to *workspace_bytes and
 * returns VX_OK. Otherwise *workspace_bytes must be at least that size.
 * The workspace holds partial results only; its contents need no setup. */
vx_status vx_sparse_decode(const vx_pages* pages, const vx_geom* geom,
                           const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* sel,
                           int32_t sel_stride, const int32_t* sel_count,
                           float sm_scale, float* out, float* lse,
                           int32_t num_splits, void* workspace,
                           size_t* workspace_bytes, hipStream_t stream);

/* The whole decode step (Vortex paper note, "System design > 1. vFlow":
 * cache stage, indexer, sparse attention; "System design > 3. Execution
 * backend": sequence-local fusion). Writes the same bits as vx_index_pages
 * followed by vx_sparse_decode with the same arguments (the latter's sel /
 * sel_count being the former's outputs). When the plan has one split per
 * (sequence, KV head) and the geometry is GQA (group of 1, 2, 4 or 8) with
 * sel_stride <= 256 and max_pages <= 4096, it is one kernel with a block per
 * (sequence, KV head) that indexes and then attends over its own selection
 * (on the matrix cores for bf16 with Dk = 128, else on the vector ALUs).
 * MLA: the scorer, then one kernel in which every split block selects its
 * sequence's pages from the scores (the first split writes sel / sel_count)
 * and attends over its share, then the split merge. Otherwise the two calls'
 * kernels run in turn.
 * workspace == NULL: writes the bytes needed to *workspace_bytes (those of
 * vx_sparse_decode, plus 4 per sequence when the plan orders the segments,
 * see vx_plan_decode) and returns VX_OK; otherwise *workspace_bytes must be
 * at least that. */
vx_status vx_decode_step(const vx_pages* pages, const vx_geom* geom,
                         const void* q, const void* k_pool,
                         const void* v_pool, float* centroids,
                         void* cent_bf16, int32_t refresh_newest,
                         float score_scale, float sm_scale, int32_t k,
                         int32_t n_sink, int32_t n_local, int32_t mode,
                         const uint32_t* rand_u32, float* scores,
                         int32_t* sel, int32_t sel_stride,
                         int32_t* sel_count, float* out, float* lse,
                         int32_t num_splits, void* workspace,
                         size_t* workspace_bytes, hipStream_t stream);

/* vx_decode_step for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments and results (the same kernels and bits) as vx_decode_step, with
 * no workspace argument: the split partials live in a 32 MiB scratch array
 * inside the library, one per device, which each device holds until the
 * process ends. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that
 * device's scratch address. A step whose partials need more than 32 MiB
 * (batch * num_q_heads * splits * (head_dim_v + 2) * 4 bytes, split steps
 * only) returns VX_ERR_WORKSPACE before any launch. Every call on one device
 * shares its scratch, so calls that overlap on one device (different streams
 * or threads) race; calls ordered on one stream do not. The scratch needs
 * no setup: a call writes every partial it reads. */
vx_status vx_decode_step_static(const vx_pages* pages, const vx_geom* geom,
                                const void* q, const void* k_pool,
                                const void* v_pool, float* centroids,
                                void* cent_bf16, int32_t refresh_newest,
                                float score_scale, float sm_scale, int32_t k,
                                int32_t n_sink, int32_t n_local, int32_t mode,
                                const uint32_t* rand_u32, float* scores,
                                int32_t* sel, int32_t sel_stride,
                                int32_t* sel_count, float* out, float* lse,
                                int32_t num_splits, hipStream_t stream);

/* One generated token per sequence, then the whole step (Vortex paper note,
 * "System design > 1. vFlow": the cache stage's statistic follows the newest
 * token; "System design > 3. Execution backend": sequence-local fusion).
 * seq_lens already count the new token; k_new [batch][Hkv][Dk] (and v_new
 * [batch][Hkv][Dv], NULL for MLA, whose values are the latent rows) hold its
 * rows in the KV dtype. Writes the same bits as vx_centroid_update(pages,
 * geom, k_pool, v_pool, first_token = -1 for every sequence, k_new, v_new,
 * centroids, cent_bf16) followed by vx_decode_step(..., refresh_newest = 0,
 * ...) with the remaining arguments. When vx_decode_step is one kernel
 * (GQA), that kernel writes the rows into the token's slot and computes the
 * page's centroid with the new key taken from k_new; otherwise the append
 * kernel runs first. The same precondition as refresh_newest = 1: no
 * sequence's newest physical page appears in another sequence's table.
 * k_pool and v_pool are written. workspace == NULL: writes the bytes needed
 * to *workspace_bytes (as for vx_decode_step) and returns VX_OK. Argument
 * errors (VX_ERR_INVALID_ARG, as for vx_decode_step, plus a NULL k_new, or a
 * NULL v_new without MLA, or a v_new with MLA, when batch > 0) are reported
 * before any launch. */
vx_status vx_append_decode_step(const vx_pages* pages, const vx_geom* geom,
                                const void* q, void* k_pool, void* v_pool,
                                const void* k_new, const void* v_new,
                                float* centroids, void* cent_bf16,
                                float score_scale, float sm_scale, int32_t k,
                                int32_t n_sink, int32_t n_local, int32_t mode,
                                const uint32_t* rand_u32, float* scores,
                                int32_t* sel, int32_t sel_stride,
                                int32_t* sel_count, float* out, float* lse,
                                int32_t num_splits, void* workspace,
                                size_t* workspace_bytes, hipStream_t stream);

/* The whole step with the Quest-style indexer (GQA only; the mechanism is
 * Quest's, the other baseline of the Vortex paper note, "Paper context" and
 * "Key results > User-side latency"). Writes the same bits as
 * vx_bound_scores (with refresh_newest), vx_topk_pages over those scores and
 * vx_sparse_decode over that selection, in that order. When the plan has one
 * split per (sequence, KV head), the keys are bf16 and sel_stride <= 256,
 * max_pages <= 4096, it is one kernel per step, the same
 * block-per-(sequence, KV head) kernel as vx_decode_step's with the bounds
 * scorer in place of the centroid scorer. workspace == NULL: writes
 * the bytes needed to *workspace_bytes (as for vx_decode_step) and
 * returns VX_OK. */
vx_status vx_bound_decode_step(const vx_pages* pages, const vx_geom* geom,
                               const void* q, const void* k_pool,
                               const void* v_pool, void* bounds,
                               int32_t refresh_newest, float score_scale,
                               float sm_scale, int32_t k, int32_t n_sink,
                               int32_t n_local, int32_t mode,
                               const uint32_t* rand_u32, float* scores,
                               int32_t* sel, int32_t sel_stride,
                               int32_t* sel_count, float* out, float* lse,
                               int32_t num_splits, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream);

/* Workload planner (Vortex paper note, "System design > 3. Execution
 * backend": plan by batch size, sequence length, layout and operator).
 * Host only: fills *plan from host sizes; num_cus <= 0 queries the current
 * device, num_splits <= 0 lets the planner choose. Sequence lengths live on
 * the device, so the length-dependent part of the plan runs there: with
 * order_segments, vx_decode_step first ranks the sequences by pages in use
 * (a one-block kernel writing the order into its workspace) and the
 * whole-step kernel's blocks take the longest segments first. */
vx_status vx_plan_decode(const vx_pages* pages, const vx_geom* geom,
                         int32_t sel_stride, int32_t num_splits,
                         int32_t num_cus, vx_plan* plan);

/* Device-side check of the page table (Vortex paper note, "System design >
 * 2. vTensor": the page-index structure) against the contract above, which
 * the other entry points assume and do not check: one kernel writes to
 * counts[0..3) (device int32, caller-owned) the number of violations of each
 * rule, all zero for a well-formed table:
 *   counts[0]  indptr out of order: indptr[0] != 0, indptr[b+1] < indptr[b],
 *              or indptr[B] != total_pages
 *   counts[1]  sequences with seq_lens[b] < 0, seq_lens[b] > capacity *
 *              page_size, or a capacity above max_pages
 *   counts[2]  page-table entries (in use or capacity) outside
 *              [0, num_pool_pages)
 * It reads indptr[0..B], seq_lens[0..B) and page_ids[0..total_pages) and
 * nothing through their values, so a corrupted table cannot make it fault.
 * Host checks as for every entry point; counts == NULL is
 * VX_ERR_INVALID_ARG. Asynchronous like the rest: the counts are valid once
 * the stream reaches them. */
vx_status vx_check_pages(const vx_pages* pages, int32_t* counts, hipStream_t stream);

const char* vx_status_string(vx_status status);
const char* vx_last_error(void);
int32_t vx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VX_H_ */
