"""CPU oracle for one block top-k sparse-attention decode step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP path.

It is a plain, slow, fp64 statement of what the step computes for ONE
sequence, following the Vortex paper note (papers.chlience.com, "Vortex:
Efficient and Programmable Sparse Attention Serving for AI Agents"), section
"System design > 1. vFlow": a query-independent cache stage keeps one key
centroid per page; the indexer multiplies the query with the centroids, keeps
the top-k pages by score, and exact softmax attention runs over the kept
pages. Section "System design > 3. Execution backend" names the radix top-k
with stochastic early termination and remapping; the approximate selection
below is this project's reading of that phrase (the pages give no mechanism).

Arrays are float64 NumPy arrays in logical page order for one sequence:

  q  [Hq][Dk]                 query of the decode step
  k  [cap][Hkv][P][Dk]        key pages (cap >= number of pages in use)
  v  [cap][Hkv][P][Dv]        value pages (MLA: None, V = k[..., :Dv])

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* page p of a sequence of L tokens holds tokens [pP, min((p+1)P, L)); the
  sequence uses ceil(L / P) pages; the centroid is the mean over valid tokens;
* query head h belongs to KV-head group h // (Hq / Hkv); a page's score for
  KV head g is scale * sum over the group's heads of q_h . centroid;
* forced pages (sink pages at the front, a local window at the back) are
  always kept and do not count against k; the other pages are ranked by
  (score descending, logical index ascending) and the first min(k, #) kept;
  the selection is reported in ascending logical order;
* the MLA scorer consumes bf16 operands: its centroids are rounded to bf16
  (round to nearest, ties to even) before scoring;
* a GQA scorer that keeps its centroids in bf16 (``score_bf16``) scores the
  bf16 rounding (nearest, ties to even) of the cache stage's fp32 centroid
  (``centroids_fp32``), the value such a store holds; the query is not
  rounded.

Parity status: the pages print no worked example, so every function here is
pinned by closed forms, invariants, brute force or an independent library
routine (tests/test_oracle_pins.py). ``topk_approx`` follows this project's
reading of an undescribed mechanism and is pinned only by the invariants its
reading implies (parity unpinned against the pages themselves).

An alternative cache stage and scorer, ``page_bounds`` and ``bound_scores``,
states the query-aware page bounds of Quest (Tang et al., "Quest:
Query-Aware Sparsity for Efficient Long-Context LLM Inference", ICML 2024),
which the Vortex paper note names as its other baseline ("Paper context",
"Key results > User-side latency"): per page the elementwise minimum and maximum of its keys,
and as the page's score an upper bound of q . k over its tokens.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "num_pages", "valid_tokens", "centroids", "round_to_bf16", "page_scores",
    "forced_pages", "topk_exact", "topk_approx", "approx_buckets",
    "attention", "decode_sequence", "page_bounds", "bound_scores", "centroids_fp32",
]


def num_pages(seq_len: int, page_size: int) -> int:
    """Pages a sequence of ``seq_len`` tokens occupies (paged KV cache)."""
    return -(-seq_len // page_size)


def valid_tokens(seq_len: int, page_size: int, p: int) -> int:
    """Tokens of logical page ``p`` that exist (the last page may be partial)."""
    return max(0, min(page_size, seq_len - p * page_size))


def centroids(k: np.ndarray, seq_len: int, page_size: int) -> np.ndarray:
    """Cache stage: the key centroid of each page in use.

    Vortex paper note, "System design > 1. vFlow": the cache stage computes a
    query-independent statistic per block, for block top-k the key centroid.
    Returns [n][Hkv][Dk] float64, n = ceil(seq_len / P), the mean over the
    page's valid tokens only.
    """
    n = num_pages(seq_len, page_size)
    Hkv, Dk = k.shape[1], k.shape[3]
    out = np.zeros((n, Hkv, Dk), dtype=np.float64)
    for p in range(n):
        nv = valid_tokens(seq_len, page_size, p)
        out[p] = k[p, :, :nv, :].astype(np.float64).sum(axis=1) / nv
    return out


def centroids_fp32(k: np.ndarray, seq_len: int, page_size: int) -> np.ndarray:
    """The cache stage in the precision this project defines for it (the
    pages fix none): per page and KV head, the valid keys added in token order
    with every addition rounded to fp32, then one IEEE fp32 division by the
    number of valid tokens. Keys must be fp32-representable (bf16 and fp32
    keys are). Returns [n][Hkv][Dk] float32."""
    n = num_pages(seq_len, page_size)
    Hkv, Dk = k.shape[1], k.shape[3]
    out = np.zeros((n, Hkv, Dk), dtype=np.float32)
    for p in range(n):
        nv = valid_tokens(seq_len, page_size, p)
        acc = np.zeros((Hkv, Dk), dtype=np.float32)
        for t in range(nv):
            acc = acc + k[p, :, t, :].astype(np.float32)  # float32 + float32: rounded
        out[p] = acc / np.float32(nv)
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even, returned as float64. Normal range only (|x| >= 2**-126 or
    0), which covers every centroid here."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def page_scores(q: np.ndarray, cent: np.ndarray, num_kv_heads: int,
                scale: float, score_dim: int = None) -> np.ndarray:
    """Indexer scoring: query times centroids.

    Vortex paper note, "System design > 1. vFlow": the indexer scores blocks
    by a matrix product of the query with the cached centroids. Heads of one
    GQA group share their KV head's pages, so the group's query heads are
    summed: s[g][p] = scale * sum_{h in group g} sum_d q[h][d] cent[p][g][d].
    ``score_dim`` (optional) keeps only the first score_dim columns of q and
    the centroids: the rope-unaware MLA indexer of "Key results > MLA" scores
    on the 512 latent columns and ignores the 64 rope columns.
    Returns [Hkv][n] float64.
    """
    if score_dim is not None:
        q = q[:, :score_dim]
        cent = cent[..., :score_dim]
    Hq = q.shape[0]
    G = Hq // num_kv_heads
    n = cent.shape[0]
    s = np.zeros((num_kv_heads, n), dtype=np.float64)
    for g in range(num_kv_heads):
        heads = q[g * G:(g + 1) * G].astype(np.float64)  # [G][Dk]
        per_head = heads @ cent[:, g, :].T  # [G][n]
        s[g] = scale * per_head.sum(axis=0)
    return s


def page_bounds(k: np.ndarray, seq_len: int, page_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Alternative cache stage (Quest's page metadata): for each page in use
    and KV head, the elementwise minimum and maximum of the page's valid
    keys. Returns (lo, hi), each [n][Hkv][Dk]."""
    n = num_pages(seq_len, page_size)
    hkv, dk = k.shape[1], k.shape[3]
    lo = np.zeros((n, hkv, dk))
    hi = np.zeros((n, hkv, dk))
    for p in range(n):
        keys = k[p, :, :valid_tokens(seq_len, page_size, p), :]  # [Hkv][nv][Dk]
        lo[p] = keys.min(axis=1)
        hi[p] = keys.max(axis=1)
    return lo, hi


def bound_scores(q: np.ndarray, lo: np.ndarray, hi: np.ndarray, num_kv_heads: int,
                 scale: float) -> np.ndarray:
    """Alternative scorer (Quest's criticality bound), for a GQA group: with
    Q the group-summed query of KV head g (the query the centroid scorer
    uses), the score of page p is scale * sum over dims d of
    max(Q_d * lo_d, Q_d * hi_d). Since lo_d <= k_d <= hi_d for every key k of
    the page, each term bounds Q_d * k_d from above, so the score bounds
    scale * Q . k for every token of the page, and is the least such bound
    that depends on lo and hi alone (the box's best corner attains it).
    Returns [Hkv][n]."""
    hq = q.shape[0]
    G = hq // num_kv_heads
    n = lo.shape[0]
    out = np.zeros((num_kv_heads, n))
    for g in range(num_kv_heads):
        Q = q[g * G:(g + 1) * G].sum(axis=0)  # [Dk]
        a = Q[None, :] * lo[:, g, :]  # [n][Dk]
        b = Q[None, :] * hi[:, g, :]
        out[g] = np.maximum(a, b).sum(axis=1)
    return out * scale


def forced_pages(n: int, n_sink: int, n_local: int) -> list[int]:
    """Pages kept regardless of score: the first ``n_sink`` pages and the last
    ``n_local`` pages (the local window ends with the page holding the newest
    token), restricted to [0, n)."""
    f = set(range(min(n_sink, n)))
    f.update(range(max(0, n - n_local), n))
    return sorted(f)


def _finish(n: int, forced: list[int], chosen, k_out: int) -> np.ndarray:
    sel = sorted(set(forced) | set(int(c) for c in chosen))
    out = np.full(k_out, -1, dtype=np.int64)
    out[:len(sel)] = sel
    return out


def topk_exact(scores: np.ndarray, k: int, n_sink: int, n_local: int) -> np.ndarray:
    """Indexer selection for one (sequence, KV head).

    Vortex paper note, "System design > 1. vFlow": keep the top-k blocks by
    score. Ranking: score descending, then lower logical page index first
    (so -0.0 and +0.0 tie). Forced pages are kept on top of the k ranked ones.
    Returns int64 [k + n_sink + n_local], ascending, padded with -1.
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    forced = forced_pages(n, n_sink, n_local)
    cand = np.array([p for p in range(n) if p not in set(forced)], dtype=np.int64)
    take = min(k, cand.shape[0])
    if take > 0:
        order = np.lexsort((cand, -scores[cand]))  # primary: -score ascending
        chosen = cand[order[:take]]
    else:
        chosen = []
    return _finish(n, forced, chosen, k + n_sink + n_local)


APPROX_BUCKET_BITS = 8


def approx_buckets(cand_scores_f32: np.ndarray) -> np.ndarray:
    """Remap step of the approximate selection (this project's reading of
    "remapping", Vortex paper note, "System design > 3. Execution backend"):
    an affine map of the candidates' fp32 scores onto 2**8 buckets, taken in
    fp32 exactly as written here: w = mx - mn; if w > 0,
    bucket = min(255, floor((s - mn) * (256 / w))), else bucket 0."""
    s = np.asarray(cand_scores_f32, dtype=np.float32)
    nb = np.float32(1 << APPROX_BUCKET_BITS)
    if s.shape[0] == 0:
        return np.zeros(0, dtype=np.int64)
    mn = np.min(s)
    mx = np.max(s)
    w = np.float32(mx - mn)
    if not (w > np.float32(0.0)):
        return np.zeros(s.shape[0], dtype=np.int64)
    inv = np.float32(nb / w)
    t = (s - mn).astype(np.float32) * inv
    b = np.floor(t.astype(np.float32)).astype(np.int64)
    return np.minimum(b, (1 << APPROX_BUCKET_BITS) - 1)


def topk_approx(scores_f32: np.ndarray, k: int, n_sink: int, n_local: int,
                rand_u32: int) -> np.ndarray:
    """Approximate selection for one (sequence, KV head): radix top-k with
    early termination and remapping, as this project reads the Vortex paper
    note ("System design > 3. Execution backend"; "kernel ablation" reports it
    by recall@k).

    1. Remap the candidates' scores onto 256 buckets (``approx_buckets``).
    2. One digit pass: count candidates per bucket; the boundary bucket t is
       the one where the count from the top first reaches k.
    3. Stop there (early termination): keep every candidate above t, and fill
       the remaining r places from bucket t stochastically: order its members
       by logical index, start at offset rand_u32 mod (members) and take r
       members cyclically.
    Forced pages are kept as in ``topk_exact``; with at most k candidates all
    are kept.
    """
    s = np.asarray(scores_f32, dtype=np.float32)
    n = s.shape[0]
    forced = forced_pages(n, n_sink, n_local)
    fs = set(forced)
    cand = np.array([p for p in range(n) if p not in fs], dtype=np.int64)
    k_out = k + n_sink + n_local
    if cand.shape[0] <= k:
        return _finish(n, forced, cand, k_out)
    if k == 0:
        return _finish(n, forced, [], k_out)
    bk = approx_buckets(s[cand])
    hist = np.bincount(bk, minlength=1 << APPROX_BUCKET_BITS)
    above = 0
    t = (1 << APPROX_BUCKET_BITS) - 1
    while above + hist[t] < k:
        above += hist[t]
        t -= 1
    r = k - above
    chosen = list(cand[bk > t])
    members = cand[bk == t]  # ascending logical index
    m = members.shape[0]
    off = int(rand_u32) % m
    for j in range(r):
        chosen.append(members[(off + j) % m])
    return _finish(n, forced, chosen, k_out)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_len: int,
              page_size: int, sel: np.ndarray, sm_scale: float,
              num_kv_heads: int) -> tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention over the selected pages.

    Vortex paper note, "System design > 1. vFlow": after selection, exact
    softmax attention runs over the chosen blocks only. ``sel`` is
    [Hkv][K_out] logical page ids (-1 = unused). For query head h (KV head
    g = h // G) the keys are the valid tokens of g's selected pages:
    z_t = sm_scale * q_h . k_t, o_h = sum_t softmax(z)_t v_t,
    lse_h = max z + ln sum_t exp(z_t - max z) (natural log).
    Returns out [Hq][Dv] and lse [Hq]; a head with no key gets zeros and
    lse = -inf.
    """
    Hq = q.shape[0]
    G = Hq // num_kv_heads
    Dv = v.shape[3]
    out = np.zeros((Hq, Dv), dtype=np.float64)
    lse = np.full(Hq, -np.inf, dtype=np.float64)
    for g in range(num_kv_heads):
        rows_k, rows_v = [], []
        for p in sel[g]:
            if p < 0:
                continue
            nv = valid_tokens(seq_len, page_size, int(p))
            rows_k.append(k[p, g, :nv, :])
            rows_v.append(v[p, g, :nv, :])
        if not rows_k:
            continue
        K = np.concatenate(rows_k, axis=0).astype(np.float64)  # [T][Dk]
        V = np.concatenate(rows_v, axis=0).astype(np.float64)  # [T][Dv]
        for h in range(g * G, (g + 1) * G):
            z = sm_scale * (K @ q[h].astype(np.float64))
            zmax = z.max()
            w = np.exp(z - zmax)
            den = w.sum()
            out[h] = (w @ V) / den
            lse[h] = zmax + math.log(den)
    return out, lse


def decode_sequence(seq: dict, *, page_size: int, num_kv_heads: int, k: int,
                    n_sink: int, n_local: int, score_scale: float,
                    sm_scale: float, mla: bool = False, head_dim_v: int = None,
                    approx: bool = False, score_dim: int = None,
                    indexer: str = "centroid", score_bf16: bool = False) -> dict:
    """The whole step for one sequence: cache stage, scoring, selection,
    attention. ``seq`` holds q, k, v (v None for MLA), seq_len and rand_u32
    ([Hkv] uint32 draws for the approximate selection); ``score_dim`` as in
    page_scores; ``indexer`` "centroid" (the method) or "bounds" (Quest's
    page bounds, GQA only); ``score_bf16`` (GQA) scores the bf16 rounding of
    the fp32 centroids (centroids_fp32) instead of the exact means."""
    q, kk, vv, L = seq["q"], seq["k"], seq["v"], seq["seq_len"]
    if mla:
        vv = kk[..., :head_dim_v]
    cent = centroids(kk, L, page_size)
    if indexer == "bounds":
        lo, hi = page_bounds(kk, L, page_size)
        scores = bound_scores(q, lo, hi, num_kv_heads, score_scale)
    else:
        if mla:
            score_cent = round_to_bf16(cent)
        elif score_bf16:
            score_cent = round_to_bf16(centroids_fp32(kk, L, page_size))
        else:
            score_cent = cent
        scores = page_scores(q, score_cent, num_kv_heads, score_scale, score_dim)
    k_out = k + n_sink + n_local
    sel = np.full((num_kv_heads, k_out), -1, dtype=np.int64)
    for g in range(num_kv_heads):
        if approx:
            sel[g] = topk_approx(scores[g].astype(np.float32), k, n_sink,
                                 n_local, int(seq["rand_u32"][g]))
        else:
            sel[g] = topk_exact(scores[g], k, n_sink, n_local)
    out, lse = attention(q, kk, vv, L, page_size, sel, sm_scale, num_kv_heads)
    r = {"centroids": cent, "scores": scores, "sel": sel, "out": out, "lse": lse}
    if indexer == "bounds":
        r["lo"], r["hi"] = lo, hi
    return r
