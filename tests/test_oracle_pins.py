"""Pins of the CPU oracle against facts other than itself.

The pages print no worked numeric example, so each oracle function is pinned
by closed forms, brute-force characterisations on tiny inputs, and library
routines that compute the same definition independently (torch's scaled
dot-product attention, scipy's logsumexp, torch's fp32->bf16 conversion).
Each pin is chosen so that a plausible slip (dividing by P instead of the
valid-token count, a wrong head-to-group map, a reversed tie-break, a missed
mask) fails it.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import vx_oracle as O


# ---------------------------------------------------------------- centroids

def _keys_equal_position(cap, Hkv, P, D, L, garbage=1e6):
    """Key of token t (every dim) = t + 1000*g; invalid slots hold garbage."""
    k = np.full((cap, Hkv, P, D), garbage)
    for p in range(cap):
        for g in range(Hkv):
            for s in range(P):
                t = p * P + s
                if t < L:
                    k[p, g, s, :] = t + 1000.0 * g
    return k


@pytest.mark.parametrize("P,L", [(16, 1024), (16, 1000), (4, 9), (64, 65), (16, 1)])
def test_centroid_closed_form_partial_last_page(P, L):
    cap = -(-L // P) + 2  # page-table headroom beyond the pages in use
    k = _keys_equal_position(cap, 2, P, 3, L)
    c = O.centroids(k, L, P)
    n = -(-L // P)
    assert c.shape == (n, 2, 3)
    for p in range(n):
        nv = min(P, L - p * P)
        first = p * P
        mean_t = first + (nv - 1) / 2.0  # mean of an arithmetic run
        for g in range(2):
            np.testing.assert_allclose(c[p, g], mean_t + 1000.0 * g, rtol=0, atol=1e-9)


def test_centroid_identical_keys_is_the_key():
    rng = np.random.default_rng(1)
    P, L = 16, 40
    key = rng.standard_normal((1, 2, 1, 8))
    k = np.broadcast_to(key, (3, 2, P, 8)).copy()
    c = O.centroids(k, L, P)
    for p in range(3):
        np.testing.assert_allclose(c[p], key[0, :, 0, :], rtol=1e-15)


# ---------------------------------------------------------------- bf16

def test_round_to_bf16_matches_torch_conversion():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).float().double().numpy()
    got = O.round_to_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_to_bf16_ties_to_even():
    s = 2.0 ** -7  # bf16 spacing on [1, 2)
    cases = {1.0 + s / 2: 1.0, 1.0 + 3 * s / 2: 1.0 + 2 * s, -(1.0 + s / 2): -1.0,
             1.0 + s / 2 + 1e-12: 1.0 + s, 0.0: 0.0, 3.0: 3.0}
    for x, want in cases.items():
        assert O.round_to_bf16(np.array([x]))[0] == want, x


# ---------------------------------------------------------------- scores

def test_scores_one_hot_query_picks_group_and_dim():
    rng = np.random.default_rng(3)
    Hq, Hkv, D, n = 6, 2, 5, 7  # G = 3: heads 0-2 -> KV head 0, 3-5 -> 1
    cent = rng.standard_normal((n, Hkv, D))
    for h in range(Hq):
        for d in (0, 3):
            q = np.zeros((Hq, D))
            q[h, d] = 1.0
            s = O.page_scores(q, cent, Hkv, 0.25)
            g = h // 3
            np.testing.assert_allclose(s[g], 0.25 * cent[:, g, d], rtol=1e-15)
            np.testing.assert_array_equal(s[1 - g], 0.0)


def test_scores_sum_over_group_heads_and_zero_query():
    rng = np.random.default_rng(4)
    Hq, Hkv, D, n = 4, 2, 8, 5
    cent = rng.standard_normal((n, Hkv, D))
    q = rng.standard_normal((Hq, D))
    s = O.page_scores(q, cent, Hkv, 1.0)
    # a group's score is additive in its heads: zero one head, add it back
    for h in range(Hq):
        qa = q.copy(); qa[h] = 0
        qb = np.zeros_like(q); qb[h] = q[h]
        np.testing.assert_allclose(O.page_scores(qa, cent, Hkv, 1.0) +
                                   O.page_scores(qb, cent, Hkv, 1.0), s, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(O.page_scores(np.zeros((Hq, D)), cent, Hkv, 1.0), 0.0)


def test_scores_latent_only_drops_exactly_the_rope_columns():
    """score_dim = 512 of 576 (the rope-unaware MLA indexer): one-hot queries
    in a latent column score as before, in a rope column score zero; with the
    query's rope columns zero the two scorers agree; score_dim = Dk is the
    plain scorer."""
    rng = np.random.default_rng(31)
    Hq, D, lat, n = 4, 576, 512, 6
    cent = rng.standard_normal((n, 1, D))
    for d in (0, 300, 511, 512, 575):
        q = np.zeros((Hq, D))
        q[2, d] = 1.0
        s = O.page_scores(q, cent, 1, 0.5, score_dim=lat)
        want = 0.5 * cent[:, 0, d] if d < lat else np.zeros(n)
        np.testing.assert_allclose(s[0], want, rtol=1e-15)
    q = rng.standard_normal((Hq, D))
    np.testing.assert_array_equal(O.page_scores(q, cent, 1, 0.5, score_dim=D),
                                  O.page_scores(q, cent, 1, 0.5))
    q[:, lat:] = 0.0
    np.testing.assert_allclose(O.page_scores(q, cent, 1, 0.5, score_dim=lat),
                               O.page_scores(q, cent, 1, 0.5), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- selection

def test_forced_pages_cases():
    assert O.forced_pages(0, 1, 1) == []
    assert O.forced_pages(1, 1, 1) == [0]
    assert O.forced_pages(2, 1, 2) == [0, 1]
    assert O.forced_pages(5, 1, 2) == [0, 3, 4]
    assert O.forced_pages(64, 0, 1) == [63]
    assert O.forced_pages(10, 0, 0) == []


def _beats(s, x, y):
    return s[x] > s[y] or (s[x] == s[y] and x < y)


@pytest.mark.parametrize("seed", range(40))
def test_topk_exact_rank_characterisation(seed):
    """Brute force: a candidate is chosen iff fewer than k candidates beat it
    (higher score, or equal score and lower index)."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 65))
    k = int(rng.integers(0, 20))
    n_sink, n_local = int(rng.integers(0, 2)), int(rng.integers(0, 3))
    s = rng.integers(-3, 4, size=n).astype(np.float64)  # many duplicates
    if seed % 3 == 0:
        s = rng.standard_normal(n)
    sel = O.topk_exact(s, k, n_sink, n_local)
    assert sel.shape == (k + n_sink + n_local,)
    got = [int(x) for x in sel if x >= 0]
    assert got == sorted(set(got))  # ascending, no repeats
    assert all(x == -1 for x in sel[len(got):])  # padding after the ids
    forced = O.forced_pages(n, n_sink, n_local)
    assert set(forced) <= set(got)
    cand = [p for p in range(n) if p not in forced]
    chosen = set(got) - set(forced)
    assert len(chosen) == min(k, len(cand))
    for c in cand:
        nbeat = sum(_beats(s, x, c) for x in cand if x != c)
        assert (c in chosen) == (nbeat < k), (c, nbeat, k)


def test_topk_exact_ties_and_signed_zero():
    s = np.zeros(10)
    assert list(O.topk_exact(s, 3, 0, 1)) == [0, 1, 2, 9]
    assert list(O.topk_exact(s, 3, 1, 1)) == [0, 1, 2, 3, 9]
    s2 = np.array([-0.0, 0.0, -0.0, 0.0])
    assert list(O.topk_exact(s2, 2, 0, 0)) == [0, 1]
    s3 = np.array([0.0, -0.0, 1.0])
    assert list(O.topk_exact(s3, 2, 0, 0)) == [0, 2]
    # k at least the candidate count -> every page
    assert list(O.topk_exact(np.arange(5.0), 9, 1, 1)) == [0, 1, 2, 3, 4] + [-1] * 6


# ---------------------------------------------------------------- approx

def test_approx_equals_exact_without_bucket_collisions():
    for n in (5, 50, 200, 257):
        s = np.arange(n, dtype=np.float32)[::-1].copy()  # one candidate per bucket
        for k in (1, 4, 16, 64):
            for rnd in (0, 7, 2**32 - 1):
                a = O.topk_approx(s, k, 1, 1, rnd)
                e = O.topk_exact(s.astype(np.float64), k, 1, 1)
                np.testing.assert_array_equal(a, e)


@pytest.mark.parametrize("seed", range(30))
def test_approx_invariants(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(2, 1100))
    k = int(rng.integers(1, 70))
    s = rng.standard_normal(n).astype(np.float32)
    if seed % 4 == 0:
        s = np.round(s * 3).astype(np.float32)  # heavy ties
    rnd = int(rng.integers(0, 2**32))
    sel = O.topk_approx(s, k, 0, 1, rnd)
    got = set(int(x) for x in sel if x >= 0)
    forced = set(O.forced_pages(n, 0, 1))
    cand = np.array([p for p in range(n) if p not in forced])
    chosen = got - forced
    assert len(chosen) == min(k, len(cand))
    if len(cand) <= k:
        return
    b = O.approx_buckets(s[cand])
    # buckets are monotone in the score
    order = np.argsort(s[cand], kind="stable")
    assert np.all(np.diff(b[order]) >= 0)
    t = min(b[np.isin(cand, list(chosen))])
    assert set(cand[b > t]) <= chosen  # everything above the boundary
    assert not (chosen & set(cand[b < t]))  # nothing below it
    members = list(cand[b == t])
    r = len(chosen & set(members))
    off = rnd % len(members)
    want = {members[(off + j) % len(members)] for j in range(r)}
    assert chosen & set(members) == want


def test_approx_recall_on_normal_scores():
    rng = np.random.default_rng(7)
    rec = []
    for _ in range(40):
        s = rng.standard_normal(1024).astype(np.float32)
        a = set(O.topk_approx(s, 64, 0, 0, int(rng.integers(0, 2**32))))
        e = set(O.topk_exact(s.astype(np.float64), 64, 0, 0))
        rec.append(len(a & e) / 64)
    assert np.mean(rec) > 0.97


# ---------------------------------------------------------------- attention

def _sdpa(q, K, V, scale):
    """torch's scaled dot-product attention, fp64 on the CPU."""
    qt = torch.from_numpy(q)[None, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None], scale=scale)
    return out[0, 0, 0].numpy()


@pytest.mark.parametrize("mla", [False, True])
def test_full_selection_equals_dense_attention(mla):
    rng = np.random.default_rng(11)
    P, L, Hkv, Hq = 8, 53, (1 if mla else 2), 4
    Dk, Dv = (12, 8) if mla else (6, 5)
    cap = -(-L // P) + 1
    q = rng.standard_normal((Hq, Dk))
    k = rng.standard_normal((cap, Hkv, P, Dk))
    v = None if mla else rng.standard_normal((cap, Hkv, P, Dv))
    n = -(-L // P)
    res = O.decode_sequence({"q": q, "k": k, "v": v, "seq_len": L,
                             "rand_u32": np.zeros(Hkv, np.uint32)},
                            page_size=P, num_kv_heads=Hkv, k=n, n_sink=1,
                            n_local=1, score_scale=0.3, sm_scale=0.7, mla=mla,
                            head_dim_v=Dv)
    vv = k[..., :Dv] if mla else v
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        K = k[:, g].reshape(cap * P, Dk)[:L]
        V = vv[:, g].reshape(cap * P, Dv)[:L]
        np.testing.assert_allclose(res["out"][h], _sdpa(q[h], K, V, 0.7), rtol=1e-12, atol=1e-12)
        z = 0.7 * K @ q[h]
        np.testing.assert_allclose(res["lse"][h], scipy.special.logsumexp(z), rtol=1e-13)


def test_attention_equal_keys_gives_mean_of_values():
    rng = np.random.default_rng(12)
    P, L = 4, 10  # pages 0,1 full, page 2 has 2 tokens
    k = np.broadcast_to(rng.standard_normal(3), (3, 1, P, 3)).copy()
    v = rng.standard_normal((3, 1, P, 2))
    v[2, 0, 2:, :] = 1e9  # invalid slots must not leak in
    q = rng.standard_normal((2, 3))
    sel = np.array([[0, 2, -1]])
    out, lse = O.attention(q, k, v, L, P, sel, 0.5, 1)
    want = np.concatenate([v[0, 0], v[2, 0, :2]]).mean(axis=0)
    for h in range(2):
        np.testing.assert_allclose(out[h], want, rtol=1e-13)
        z = 0.5 * float(k[0, 0, 0] @ q[h])
        np.testing.assert_allclose(lse[h], z + math.log(6), rtol=1e-13)


def test_attention_single_token_and_empty_selection():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((1, 1, 16, 4))
    v = rng.standard_normal((1, 1, 16, 3))
    q = rng.standard_normal((1, 4))
    out, lse = O.attention(q, k, v, 1, 16, np.array([[0]]), 1.0, 1)
    np.testing.assert_array_equal(out[0], v[0, 0, 0])
    np.testing.assert_allclose(lse[0], float(k[0, 0, 0] @ q[0]), rtol=1e-15)
    out, lse = O.attention(q, k, v, 1, 16, np.array([[-1]]), 1.0, 1)
    assert np.all(out == 0) and lse[0] == -np.inf


def test_hand_worked_example():
    """Worked by hand: P=2, L=5, Hq=2, Hkv=1, D=2, scale 1, sm_scale 1.
    keys t0..t4 = (1,0) (3,0) | (0,2) (0,4) | (-2,-2)
      centroids: page0 (2,0), page1 (0,3), page2 (-2,-2) (one valid token)
    q = h0 (1,0), h1 (0,1): group sum (1,1) -> scores 2, 3, -4
    k=1 ranked page + last page: candidates {0,1} -> page 1; sel = [1, 2]
    values t2 (1,0), t3 (-1,0), t4 (0,5)
    h0 logits over t2,t3,t4 = 0, 0, -2 -> out = (0, 5e^-2) / (2 + e^-2)
    h1 logits = 2, 4, -2 -> weights e^2, e^4, e^-2
    """
    k = np.zeros((3, 1, 2, 2)); v = np.zeros((3, 1, 2, 2))
    keys = [(1, 0), (3, 0), (0, 2), (0, 4), (-2, -2)]
    vals = [(9, 9), (9, 9), (1, 0), (-1, 0), (0, 5)]
    for t in range(5):
        k[t // 2, 0, t % 2] = keys[t]
        v[t // 2, 0, t % 2] = vals[t]
    k[2, 0, 1] = (50, 50)  # invalid slot
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    r = O.decode_sequence({"q": q, "k": k, "v": v, "seq_len": 5,
                           "rand_u32": np.zeros(1, np.uint32)}, page_size=2,
                          num_kv_heads=1, k=1, n_sink=0, n_local=1,
                          score_scale=1.0, sm_scale=1.0)
    np.testing.assert_allclose(r["centroids"][:, 0], [[2, 0], [0, 3], [-2, -2]])
    np.testing.assert_allclose(r["scores"][0], [2, 3, -4])
    assert list(r["sel"][0]) == [1, 2]
    e = math.exp
    np.testing.assert_allclose(r["out"][0], [0, 5 * e(-2) / (2 + e(-2))], rtol=1e-14)
    den = e(2) + e(4) + e(-2)
    np.testing.assert_allclose(r["out"][1], [(e(2) - e(4)) / den, 5 * e(-2) / den], rtol=1e-14)
    np.testing.assert_allclose(r["lse"][1], math.log(den), rtol=1e-14)


def test_approx_buckets_closed_form():
    # w = 4 -> 256 / 4 = 64 buckets per unit; the maximum clamps to 255
    np.testing.assert_array_equal(
        O.approx_buckets(np.array([0, 1, 2, 3, 4], np.float32)), [0, 64, 128, 192, 255])
    np.testing.assert_array_equal(
        O.approx_buckets(np.array([-1.0, -0.75, -0.5, 1.0], np.float32)), [0, 32, 64, 255])
    np.testing.assert_array_equal(O.approx_buckets(np.full(7, 2.5, np.float32)), 0)


# ---------------------------------------------- page bounds (Quest-style indexer)

def test_page_bounds_brute_force_and_garbage_ignored():
    """min/max over the valid tokens of each page, taken element by element
    with Python's own min/max; slots past the last token hold garbage that
    must not leak in."""
    rng = np.random.default_rng(5)
    P, L, Hkv, D = 4, 10, 2, 3
    k = rng.standard_normal((4, Hkv, P, D))
    k[2, :, 2:, :] = 1e9   # page 2 holds 2 tokens; the rest is garbage
    k[3] = -1e9            # capacity page, not in use
    lo, hi = O.page_bounds(k, L, P)
    assert lo.shape == (3, Hkv, D)
    for p in range(3):
        nv = min(P, L - p * P)
        for g in range(Hkv):
            for d in range(D):
                col = [k[p, g, t, d] for t in range(nv)]
                assert lo[p, g, d] == min(col) and hi[p, g, d] == max(col)


def test_bound_scores_is_best_corner_of_the_box():
    """The score equals the largest group-summed logit over the 2^D corners
    of the page's min/max box (a linear function's maximum over a box sits
    at a corner), found here by enumeration."""
    import itertools
    rng = np.random.default_rng(6)
    Hq, Hkv, D, n = 4, 2, 4, 3
    q = rng.standard_normal((Hq, D))
    lo = rng.standard_normal((n, Hkv, D))
    hi = lo + rng.random((n, Hkv, D))
    s = O.bound_scores(q, lo, hi, Hkv, 0.5)
    for g in range(Hkv):
        for p in range(n):
            best = -np.inf
            for bits in itertools.product((0, 1), repeat=D):
                c = np.where(np.array(bits) == 1, hi[p, g], lo[p, g])
                val = sum(float(q[h] @ c) for h in (2 * g, 2 * g + 1))
                best = max(best, val)
            np.testing.assert_allclose(s[g, p], 0.5 * best, rtol=1e-13)


def test_bound_scores_bounds_every_token_and_is_exact_for_one_token():
    """Upper bound of scale * sum_h q_h . k over every valid token; a page
    with a single valid token scores exactly its logit."""
    rng = np.random.default_rng(7)
    P, L, Hq, Hkv, D = 8, 41, 6, 2, 16
    k = rng.standard_normal((6, Hkv, P, D))
    q = rng.standard_normal((Hq, D))
    lo, hi = O.page_bounds(k, L, P)
    s = O.bound_scores(q, lo, hi, Hkv, 0.25)
    n = -(-L // P)
    for g in range(Hkv):
        for p in range(n):
            nv = min(P, L - p * P)
            logits = [0.25 * sum(float(q[h] @ k[p, g, t]) for h in range(3 * g, 3 * g + 3))
                      for t in range(nv)]
            assert s[g, p] >= max(logits) - 1e-12
            if nv == 1:
                np.testing.assert_allclose(s[g, p], logits[0], rtol=1e-13)
    assert L % P == 1  # the last page holds one token


def test_bound_scores_hand_worked():
    """Worked by hand, one head: q = (1, -1); page keys (0, 1), (2, -1) ->
    lo (0, -1), hi (2, 1); bound max(0, 2) + max(1, -1) = 3, attained by the
    key (2, -1). Keys (1, 0), (0, 1) with q = (1, 1): box corner (1, 1)
    gives 2 though no key exceeds 1 (the bound is loose there)."""
    k = np.zeros((2, 1, 2, 2))
    k[0, 0, 0], k[0, 0, 1] = (0, 1), (2, -1)
    k[1, 0, 0], k[1, 0, 1] = (1, 0), (0, 1)
    lo, hi = O.page_bounds(k, 4, 2)
    np.testing.assert_array_equal(lo[0, 0], [0, -1])
    np.testing.assert_array_equal(hi[0, 0], [2, 1])
    assert O.bound_scores(np.array([[1.0, -1.0]]), lo[:1], hi[:1], 1, 1.0)[0, 0] == 3.0
    assert O.bound_scores(np.array([[1.0, 1.0]]), lo[1:], hi[1:], 1, 1.0)[0, 0] == 2.0


def test_decode_sequence_bounds_indexer():
    """indexer="bounds" ranks pages by the bound: a page whose keys straddle
    the query direction beats one whose mean is higher but whose keys are
    all alike. P=2, L=6, one head, q = (1, 0), k=1, no forced pages."""
    k = np.zeros((3, 1, 2, 2))
    k[0, 0, 0], k[0, 0, 1] = (1, 0), (1, 0)     # mean 1, max 1
    k[1, 0, 0], k[1, 0, 1] = (3, 0), (-2.5, 0)  # mean 0.25, max 3
    k[2, 0, 0], k[2, 0, 1] = (0, 0), (0, 0)
    v = np.ones((3, 1, 2, 2))
    seq = {"q": np.array([[1.0, 0.0]]), "k": k, "v": v, "seq_len": 6,
           "rand_u32": np.zeros(1, np.uint32)}
    kw = dict(page_size=2, num_kv_heads=1, k=1, n_sink=0, n_local=0, score_scale=1.0,
              sm_scale=1.0)
    cent = O.decode_sequence(seq, **kw)
    bnd = O.decode_sequence(seq, indexer="bounds", **kw)
    assert list(cent["sel"][0]) == [0]
    assert list(bnd["sel"][0]) == [1]
    np.testing.assert_allclose(bnd["scores"][0], [1, 3, 0])


# ------------------------------------------- the cache stage's fp32 definition

def test_centroids_fp32_token_order():
    """Addition in token order with fp32 rounding after each step: keys
    2**24, 1, 1 sum to 2**24 (each +1 rounds away: ties to even), while any
    order that adds the ones first gives 2**24 + 2; the mean is then one fp32
    division of 2**24 by 3."""
    k = np.zeros((1, 1, 4, 1))
    k[0, 0, :3, 0] = [2.0 ** 24, 1.0, 1.0]
    c = O.centroids_fp32(k, 3, 4)
    assert c.dtype == np.float32
    assert c[0, 0, 0] == np.float32(2.0 ** 24) / np.float32(3)
    assert c[0, 0, 0] != np.float32((2.0 ** 24 + 2) / 3)


def test_centroids_fp32_matches_fp64_when_exact():
    """Small integer keys sum exactly in fp32, so the fp32 centroid is the
    fp64 one rounded once; a partial last page divides by its own count."""
    rng = np.random.default_rng(11)
    P, L = 16, 45
    k = rng.integers(-50, 51, size=(4, 2, P, 8)).astype(np.float64)
    c32 = O.centroids_fp32(k, L, P)
    c64 = O.centroids(k, L, P)
    np.testing.assert_array_equal(c32, c64.astype(np.float32))
    assert c32.shape == (3, 2, 8)


def test_decode_sequence_bf16_centroid_scores():
    """score_bf16: each score is the fp32-summed query (not rounded) times
    the bf16 rounding of the fp32 token-order centroid. P=3, L=6, two query
    heads of 1 + 2**-12 on dim 0 (sum 2 + 2**-11). Page 0's keys
    1 + 2**-8 (twice) and 1 + 2**-8 + 2**-23 sum in fp32 to 3 + 3 * 2**-8
    (the last addition ties and rounds to even), so the fp32 centroid is
    1 + 2**-8, halfway between the bf16 values 1 and 1 + 2**-7, and rounds
    to even: 1.0; the exact mean lies above that midpoint and would round up.
    Page 1's mean 1 + 3 * 2**-9 is exact and rounds to the nearest bf16,
    1 + 2**-7."""
    k = np.zeros((2, 1, 3, 2))
    k[0, 0, :, 0] = [1 + 2.0 ** -8, 1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -23]
    k[1, 0, :, 0] = [1.0, 1.0, 1 + 9 * 2.0 ** -9]
    q = np.zeros((2, 2))
    q[:, 0] = 1 + 2.0 ** -12
    seq = {"q": q, "k": k, "v": np.ones((2, 1, 3, 2)), "seq_len": 6,
           "rand_u32": np.zeros(1, np.uint32)}
    kw = dict(page_size=3, num_kv_heads=1, k=1, n_sink=0, n_local=0, score_scale=1.0,
              sm_scale=1.0)
    r = O.decode_sequence(seq, score_bf16=True, **kw)
    qs = 2 + 2.0 ** -11
    assert r["scores"][0, 0] == qs * 1.0
    assert r["scores"][0, 1] == qs * (1 + 2.0 ** -7)
    assert list(r["sel"][0]) == [1]
    mean64 = O.centroids(k, 6, 3)[0, 0, 0]
    assert mean64 > 1 + 2.0 ** -8 and O.round_to_bf16(np.array([mean64]))[0] == 1 + 2.0 ** -7
    assert O.centroids_fp32(k, 6, 3)[0, 0, 0] == np.float32(1 + 2.0 ** -8)
