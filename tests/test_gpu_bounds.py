"""The Quest-style indexer (page bounds as the cache stage, their upper-bound
page scores) against the oracle: bounds exact, scores within the stated
tolerance, the whole step (bound scores with the newest-page refresh, top-k,
attention) matching the oracle's step with indexer="bounds"; and the refresh
paths equal a rebuild bit for bit."""

import numpy as np
import pytest
import torch

import vx_testlib as T
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

GQA_SMALL = ["tiny_fp32", "gqa_small", "longgen_small", "large_small"]


def used(w):
    return torch.from_numpy(w.page_ids.astype(np.int64)).to(w.device)


def check_against_oracle(w, step, sample, selection=True):
    """Bounds, scores, selection and attention of the sampled sequences;
    returns the number of (sequence, KV head) selections that differ from the
    oracle's within its near-tie allowance (their attention is not compared)."""
    out = step.out.cpu().double().numpy()
    lse = step.lse.cpu().double().numpy()
    G = w.spec.num_q_heads // w.spec.num_kv_heads
    differing = 0
    for b in sample:
        r = T.oracle_seq(w, step, b)
        T.check_bounds(w, step, b, r)
        T.check_bound_scores(w, step, b, r)
        if not selection:
            continue
        for g, ok in enumerate(T.check_selection(w, step, b, r)):
            if ok:
                T.check_attention(w, out[b], lse[b], r["out"], r["lse"],
                                  heads=range(g * G, (g + 1) * G), tag=f"b={b} g={g}")
            else:
                differing += 1
                T.check_attention_on_gpu_selection(w, step, b, r, out[b], lse[b], g,
                                                   tag=f"b={b} g={g}")
    return differing


@pytest.mark.parametrize("name", GQA_SMALL)
def test_rebuild_and_scores_match_oracle(name):
    w = on_gpu(W.make(SMALL[name], "cpu", seed=31))
    step = DecodeStep(w, indexer="bounds")
    step.bounds.fill_(7)
    step.rebuild_bounds()
    step.bound_score()
    T.sync()
    check_against_oracle(w, step, range(w.batch), selection=False)
    # capacity entries past a sequence's pages in use hold zeros
    for b in range(w.batch):
        lo, hi = int(w.indptr[b]), int(w.indptr[b + 1])
        ids = w.page_ids[lo + w.n_pages(b):hi]
        if len(ids):
            t = step.bounds[torch.from_numpy(ids.astype(np.int64)).to(w.device)]
            assert (t == 0).all()


@pytest.mark.parametrize("name", GQA_SMALL)
def test_step_matches_oracle(name):
    """run(): bound scores with the newest-page refresh, top-k, attention,
    after appends, against the oracle for every sequence."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=32))
    step = DecodeStep(w, indexer="bounds")
    step.rebuild_bounds()
    for _ in range(5):
        w.append_token()
        step.run()
    T.sync()
    differing = check_against_oracle(w, step, range(w.batch))
    assert differing <= max(1, w.batch * w.spec.num_kv_heads // 20)


@pytest.mark.parametrize("name", GQA_SMALL)
def test_refresh_paths_equal_rebuild(name):
    """After appends (crossing page boundaries): the scorer's fused refresh,
    vx_bounds_update with first_token -1, and a full rebuild give the same
    bounds and scores bit for bit; so do other first_token values."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=33))
    fused = DecodeStep(w, indexer="bounds")
    upd = DecodeStep(w, indexer="bounds")
    reb = DecodeStep(w, indexer="bounds")
    fused.rebuild_bounds()
    upd.rebuild_bounds()
    ids = used(w)
    B = w.batch
    for i in range(20):
        w.append_token()
        fused.bound_score(refresh=True)
        if i % 3 == 0:
            ft = torch.tensor([[0, 5, -1, -17, 10 ** 6][b % 5] for b in range(B)],
                              dtype=torch.int32, device=w.device)
            upd.refresh_bounds(first_token=ft)
        else:
            upd.refresh_bounds()
        upd.bound_score()
        reb.rebuild_bounds()
        reb.bound_score()
        T.sync()
        assert torch.equal(fused.bounds[ids], reb.bounds[ids])
        assert torch.equal(upd.bounds[ids], reb.bounds[ids])
        valid = torch.zeros(w.nnz, dtype=torch.bool)
        for b in range(B):
            lo = int(w.indptr[b])
            valid[lo:lo + w.n_pages(b)] = True
        valid = valid.to(w.device)
        assert torch.equal(fused.scores[:, valid], reb.scores[:, valid])
        assert torch.equal(upd.scores[:, valid], reb.scores[:, valid])


@pytest.mark.parametrize("k,n_sink,n_local", [(0, 1, 1), (3, 0, 0), (200, 1, 1), (5, 2, 0)])
def test_budgets(k, n_sink, n_local):
    w = on_gpu(W.make(SMALL["gqa_small"].replace(headroom_tokens=20), "cpu", seed=34))
    step = DecodeStep(w, indexer="bounds", k=k, n_sink=n_sink, n_local=n_local)
    step.rebuild_bounds()
    w.append_token()
    step.run()
    T.sync()
    assert check_against_oracle(w, step, range(w.batch)) <= max(1, w.batch // 20)


def test_idle_and_single_token_sequences():
    """seq_lens 0 (empty selection, zero output), one token, a page and a
    token: against the oracle."""
    lens = (0, 1, 16, 17, 0, 333)
    sp = W.spec("gqa_bf16", batch=len(lens), lengths=("list", lens), headroom_tokens=16,
                pool=("factor", 1.5))
    w = on_gpu(W.make(sp, "cpu", seed=35))
    step = DecodeStep(w, indexer="bounds")
    step.out.fill_(1.0)
    step.rebuild_bounds()
    step.run()
    T.sync()
    for b, L in enumerate(w.seq_lens):
        if L == 0:
            assert (step.sel_count[b] == 0).all()
            assert (step.out[b] == 0).all()
            assert torch.isneginf(step.lse[b]).all()
    assert check_against_oracle(w, step, [b for b, L in enumerate(w.seq_lens) if L]) == 0


@pytest.mark.parametrize("name,sample", [("gqa_bf16", (0, 7, 31)), ("largebatch_bf16", (3, 200))])
def test_full_size_sampled(name, sample):
    """The shapes the step is timed at: sampled sequences against the oracle."""
    w = W.make(W.spec(name, headroom_tokens=64), "cuda", seed=36)
    step = DecodeStep(w, indexer="bounds")
    step.rebuild_bounds()
    w.append_token()
    step.run()
    T.sync()
    assert check_against_oracle(w, step, sample) <= 1
    del w, step
    torch.cuda.empty_cache()


def bound_step_vs_calls(w, num_splits=0, appends=2, **kw):
    """vx_bound_decode_step against vx_bound_scores + vx_topk_pages +
    vx_sparse_decode on separate buffers: the same bits."""
    sep = DecodeStep(w, indexer="bounds", fused=False, num_splits=num_splits, **kw)
    one = DecodeStep(w, indexer="bounds", fused=True, num_splits=num_splits, **kw)
    sep.rebuild_bounds()
    one.rebuild_bounds()
    ids = used(w)
    for _ in range(appends):
        if w.spec.headroom_tokens > 0:
            w.append_token()
        valid = torch.zeros(w.nnz, dtype=torch.bool)
        for b in range(w.batch):
            lo = int(w.indptr[b])
            valid[lo:lo + w.n_pages(b)] = True
        valid = valid.to(w.device)
        sep.run()
        one.run()
        T.sync()
        assert torch.equal(sep.bounds[ids], one.bounds[ids])
        assert torch.equal(sep.scores[:, valid], one.scores[:, valid])
        assert torch.equal(sep.sel_count, one.sel_count)
        assert torch.equal(sep.sel, one.sel)
        assert torch.equal(sep.out, one.out)
        assert torch.equal(sep.lse, one.lse)
    return one


@pytest.mark.parametrize("num_splits", [0, 1])
@pytest.mark.parametrize("name", GQA_SMALL)
def test_small_bound_step_equals_calls(name, num_splits):
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=38))
    one = bound_step_vs_calls(w, num_splits=num_splits)
    spec = w.spec
    fused = one.plan()["num_splits"] == 1 and one.k_out <= 256
    assert one.plan()["fused_step"] == int(fused)  # the centroid step's plan; bounds: bf16 only


@pytest.mark.parametrize("k,n_sink,n_local", [(0, 1, 1), (3, 0, 0), (200, 1, 1), (5, 0, 3)])
def test_bound_step_budgets(k, n_sink, n_local):
    """The whole-step kernel selects inside the attention kernel: other
    budgets give the separate calls' bits and the oracle's attention."""
    w = on_gpu(W.make(SMALL["gqa_small"].replace(headroom_tokens=20), "cpu", seed=39))
    one = bound_step_vs_calls(w, num_splits=1, appends=1, k=k, n_sink=n_sink, n_local=n_local)
    assert check_against_oracle(w, one, range(w.batch)) <= max(1, w.batch // 20)


@pytest.mark.parametrize("name", ["gqa_bf16", "largebatch_bf16", "longgen_bf16"])
def test_full_size_bound_step_equals_calls(name):
    w = W.make(W.spec(name, headroom_tokens=max(64, W.spec(name).headroom_tokens)), "cuda", seed=3)
    one = bound_step_vs_calls(w)
    assert one.plan()["fused_step"] == 1
    del w, one
    torch.cuda.empty_cache()


# (Hq, Hkv, Dk, dtype): units per row C = Hkv * Dk / 4 of 512 (8 per lane), 128 (2), 64 and 32
# (1, lanes idle); group sizes 3 (no compiled group size), 2, 1 and 8.
GEOMETRIES = [(48, 16, 128, "bf16"), (8, 4, 128, "bf16"), (4, 4, 64, "bf16"), (16, 2, 64, "f32")]


@pytest.mark.parametrize("hq,hkv,dk,dt", GEOMETRIES)
def test_geometries(hq, hkv, dk, dt):
    """Other row widths and group sizes: bounds exact and scores within
    tolerance after appends; the whole step against the oracle where the
    attention takes the group size (a group of 3 runs the cache stage and the
    scorer only, through the C ABI directly)."""
    from types import SimpleNamespace
    from sparse_attention_decode_amd import binding as V
    sp = W.spec("gqa_bf16", batch=4, num_q_heads=hq, num_kv_heads=hkv, head_dim_k=dk,
                head_dim_v=dk, kv_dtype=dt, q_dtype=dt, lengths=("list", (100, 333, 17, 1)),
                headroom_tokens=24)
    w = on_gpu(W.make(sp, "cpu", seed=40))
    if hq // hkv in (1, 2, 4, 8):
        step = DecodeStep(w, indexer="bounds")
        step.rebuild_bounds()
        for _ in range(3):
            w.append_token()
            step.run()
        T.sync()
        assert check_against_oracle(w, step, range(w.batch)) <= 1
        return
    score_scale, sm_scale = sp.scales()
    pages = V.make_pages(sp.batch, sp.page_size, w.pool_pages, w.nnz, w.max_pages, w.d_indptr,
                         w.d_page_ids, w.d_seq_lens)
    geom = V.make_geom(hq, hkv, dk, dk, 0, w.q.dtype, w.k_pool.dtype, 0)
    st = SimpleNamespace(k=sp.topk, n_sink=sp.n_sink, n_local=sp.n_local, score_scale=score_scale,
                         sm_scale=sm_scale, score_dim=0, indexer="bounds",
                         bounds=torch.zeros((w.pool_pages, hkv, dk // 4, 2, 4), dtype=w.k_pool.dtype,
                                            device=w.device),
                         scores=torch.zeros((hkv, w.nnz), dtype=torch.float32, device=w.device))
    V.vx_bounds_update(pages, geom, w.k_pool, None, st.bounds)
    for _ in range(3):
        w.append_token()
        V.vx_bound_scores(pages, geom, w.q, w.k_pool, st.bounds, True, score_scale, st.scores)
    T.sync()
    for b in range(w.batch):
        r = T.oracle_seq(w, st, b)
        T.check_bounds(w, st, b, r)
        T.check_bound_scores(w, st, b, r)


@pytest.mark.parametrize("name", ["gqa_small", "large_small"])
def test_bound_step_approx_topk_equals_calls(name):
    """The approximate top-k inside the whole-step kernel gives the separate
    calls' bits on bound scores too."""
    from sparse_attention_decode_amd import binding as V
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=20), "cpu", seed=42))
    bound_step_vs_calls(w, num_splits=1, appends=2, mode=V.VX_TOPK_APPROX)


def test_bound_step_very_large_capacity():
    """Page capacity beyond the whole-step kernel's 4096 pages: the separate
    kernels run, and match the oracle."""
    sp = W.spec("gqa_bf16", batch=2, num_q_heads=4, num_kv_heads=2,
                lengths=("list", (3000, 70)), headroom_tokens=130000)
    w = W.make(sp, "cuda", seed=43)
    assert w.max_pages > 8000
    one = bound_step_vs_calls(w, appends=1)
    assert one.plan()["fused_step"] == 0
    assert check_against_oracle(w, one, range(2)) == 0
    del w, one
    torch.cuda.empty_cache()


def test_zero_query_selects_lowest_indices():
    """q = 0: every bound score is a (signed) zero, all rank equal, and the
    tie-break keeps the lowest logical pages besides the forced ones."""
    sp = W.spec("gqa_bf16", batch=3, lengths=("list", (300, 517, 64)))
    w = on_gpu(W.make(sp, "cpu", seed=5))
    w.q.zero_()
    step = DecodeStep(w, indexer="bounds")
    step.rebuild_bounds()
    step.run()
    T.sync()
    assert check_against_oracle(w, step, range(3)) == 0
    sel = step.sel.cpu().numpy()
    for b in range(3):
        n = w.n_pages(b)
        for g in range(w.spec.num_kv_heads):
            want = sorted(set(range(min(n, 1 + 16))) | {n - 1})
            assert list(sel[b, g][:len(want)]) == want
