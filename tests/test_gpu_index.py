"""The fused indexer (vx_index_pages) against the separate calls it stands
for: newest-page refresh (vx_centroid_update, first token -1), scores
(vx_page_scores) and selection (vx_topk_pages) must give the same bits, in
both top-k modes, for every geometry; and the whole step through it must
match the oracle."""

import numpy as np
import pytest
import torch

import vx_testlib as T
from sparse_attention_decode_amd import binding as V
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def used_pages(w):
    return torch.from_numpy(w.page_ids.astype(np.int64)).to(w.device)


def valid_entries(w):
    """Page-table entries holding at least one token."""
    m = np.zeros(w.nnz, dtype=bool)
    for b in range(w.batch):
        lo = int(w.indptr[b])
        m[lo:lo + w.n_pages(b)] = True
    return torch.from_numpy(m).to(w.device)


def fused_vs_separate(w, mode=V.VX_TOPK_EXACT, appends=1, **kw):
    """Grow every sequence by `appends` tokens; after each, run the separate
    calls on one set of buffers and the fused call on another; compare."""
    sep = DecodeStep(w, mode=mode, fused=False, **kw)
    fus = DecodeStep(w, mode=mode, fused=True, **kw)
    sep.rebuild_centroids()
    fus.rebuild_centroids()
    used, valid = used_pages(w), valid_entries(w)
    for _ in range(appends):
        if appends > 1 or w.spec.headroom_tokens > 0:
            w.append_token()
            valid = valid_entries(w)
        sep.refresh_centroids()
        sep.score()
        sep.select()
        fus.index()
        T.sync()
        assert torch.equal(sep.centroids[used], fus.centroids[used])
        if w.spec.mla:
            assert torch.equal(sep.cent_bf16[used], fus.cent_bf16[used])
        assert torch.equal(sep.scores[:, valid], fus.scores[:, valid])
        assert torch.equal(sep.sel_count, fus.sel_count)
        assert torch.equal(sep.sel, fus.sel)
    return sep, fus


@pytest.mark.parametrize("mode", [V.VX_TOPK_EXACT, V.VX_TOPK_APPROX])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_fused_equals_separate(name, mode):
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=11))
    fused_vs_separate(w, mode=mode, appends=3)


@pytest.mark.parametrize("name", ["gqa_bf16", "longgen_bf16", "largebatch_bf16", "mla_bf16"])
def test_full_size_fused_equals_separate(name):
    w = W.make(W.spec(name, headroom_tokens=max(64, W.spec(name).headroom_tokens)), "cuda", seed=1)
    fused_vs_separate(w, appends=2)
    del w
    torch.cuda.empty_cache()


def test_large_capacity():
    """Page capacities in the thousands (one sequence of 30000 tokens among
    short ones): same bits as the separate calls, and the oracle."""
    sp = W.spec("gqa_bf16", batch=3, num_q_heads=4, num_kv_heads=2,
                lengths=("list", (3000, 30000, 70)), headroom_tokens=16000)
    w = W.make(sp, "cuda", seed=12)
    assert w.max_pages > 2500
    fused_vs_separate(w, appends=2)
    step = DecodeStep(w)
    step.rebuild_centroids()
    step.run()
    T.sync()
    check_step_against_oracle(w, step, range(3))


def test_very_large_capacity():
    """A page capacity of ~8200 pages (beyond the whole-step kernel's 4096):
    the indexer and attention kernels give the same bits as the separate
    calls, and match the oracle."""
    sp = W.spec("gqa_bf16", batch=2, num_q_heads=4, num_kv_heads=2,
                lengths=("list", (3000, 70)), headroom_tokens=130000)
    w = W.make(sp, "cuda", seed=13)
    assert w.max_pages > 8000
    fused_vs_separate(w, appends=1)
    step = DecodeStep(w)
    step.rebuild_centroids()
    step.run()
    T.sync()
    check_step_against_oracle(w, step, range(2))
    del w, step
    torch.cuda.empty_cache()


def check_step_against_oracle(w, step, sample):
    out = step.out.cpu().double().numpy()
    lse = step.lse.cpu().double().numpy()
    G = w.spec.num_q_heads // w.spec.num_kv_heads
    differing = 0
    for b in sample:
        r = T.oracle_seq(w, step, b)
        T.check_centroids(w, step, b, r)
        T.check_scores(w, step, b, r)
        for g, ok in enumerate(T.check_selection(w, step, b, r)):
            if ok:
                T.check_attention(w, out[b], lse[b], r["out"], r["lse"],
                                  heads=range(g * G, (g + 1) * G), tag=f"b={b} g={g}")
            else:
                differing += 1
                T.check_attention_on_gpu_selection(w, step, b, r, out[b], lse[b], g,
                                                   tag=f"b={b} g={g}")
    return differing


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_step_matches_oracle(name):
    """run(): fused indexer then attention, after appends, against the oracle."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=20), "cpu", seed=13))
    step = DecodeStep(w)
    step.rebuild_centroids()
    for _ in range(5):
        w.append_token()
        step.run()
    T.sync()
    differing = check_step_against_oracle(w, step, range(w.batch))
    assert differing <= max(1, w.batch * w.spec.num_kv_heads // 20)


@pytest.mark.parametrize("headroom", [0, 16])
@pytest.mark.parametrize("base", ["gqa_bf16", "mla_bf16", "tiny_fp32"])
def test_idle_slots(base, headroom):
    """seq_lens 0 (with and without page capacity): empty selection, zero
    output, lse -inf; the other sequences are unaffected."""
    lens = (0, 40, 0, 0, 333, 0) if base != "tiny_fp32" else (0, 0, 500)
    sp = W.spec(base, batch=len(lens), lengths=("list", lens), headroom_tokens=headroom,
                pool=("factor", 1.5))
    w = on_gpu(W.make(sp, "cpu", seed=14))
    for fused in (False, True):
        step = DecodeStep(w, fused=fused)
        step.sel.fill_(7)
        step.sel_count.fill_(7)
        step.out.fill_(1.0)
        step.rebuild_centroids()
        if fused:
            step.index(refresh=False)
        else:
            step.score()
            step.select()
        step.attend()
        T.sync()
        for b, L in enumerate(lens):
            if L == 0:
                assert (step.sel_count[b] == 0).all()
                assert (step.sel[b] == -1).all()
                assert (step.out[b] == 0).all()
                assert torch.isneginf(step.lse[b]).all()
        assert check_step_against_oracle(w, step, [b for b, L in enumerate(lens) if L]) == 0


# ---- vx_decode_step: the whole step in one call ---------------------------

def step_vs_calls(w, num_splits=0, mode=V.VX_TOPK_EXACT, appends=2, **kw):
    """vx_decode_step against vx_centroid_update + vx_page_scores +
    vx_topk_pages + vx_sparse_decode on separate buffers: same bits."""
    sep = DecodeStep(w, mode=mode, fused=False, num_splits=num_splits, **kw)
    one = DecodeStep(w, mode=mode, fused=True, num_splits=num_splits, **kw)
    sep.rebuild_centroids()
    one.rebuild_centroids()
    used = used_pages(w)
    for _ in range(appends):
        if w.spec.headroom_tokens > 0:
            w.append_token()
        valid = valid_entries(w)
        sep.run()
        one.run()
        T.sync()
        assert torch.equal(sep.centroids[used], one.centroids[used])
        if sep.cent_bf16 is not None:
            assert torch.equal(sep.cent_bf16[used], one.cent_bf16[used])
        assert torch.equal(sep.scores[:, valid], one.scores[:, valid])
        assert torch.equal(sep.sel_count, one.sel_count)
        assert torch.equal(sep.sel, one.sel)
        assert torch.equal(sep.out, one.out)
        assert torch.equal(sep.lse, one.lse)
    return one


@pytest.mark.parametrize("num_splits", [0, 1])
@pytest.mark.parametrize("mode", [V.VX_TOPK_EXACT, V.VX_TOPK_APPROX])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_decode_step_equals_calls(name, mode, num_splits):
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=15))
    one = step_vs_calls(w, num_splits=num_splits, mode=mode)
    spec = w.spec
    fused = one.plan()["num_splits"] == 1 and not spec.mla and one.k_out <= 256
    assert one.plan()["fused_step"] == int(fused)


@pytest.mark.parametrize("name,fused", [("gqa_bf16", 1), ("largebatch_bf16", 1),
                                        ("longgen_bf16", 1), ("mla_bf16", 0)])
def test_full_size_decode_step_equals_calls(name, fused):
    sp = W.spec(name, headroom_tokens=max(64, W.spec(name).headroom_tokens))
    w = W.make(sp, "cuda", seed=2)
    one = step_vs_calls(w)
    assert one.plan()["fused_step"] == fused
    del w, one
    torch.cuda.empty_cache()


@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("name", ["gqa_small", "large_small", "longgen_small"])
def test_small_bf16_centroid_step_equals_calls(name, num_splits):
    """Scores on the centroids' bf16 copy: the whole-step kernel (one
    split), the fused indexer (three splits: vx_index_pages then the
    attention) and the separate calls (vx_page_scores on the copy) give the
    same bits, and match the oracle's bf16-centroid reading."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=25))
    one = step_vs_calls(w, num_splits=num_splits, score_bf16=True)
    assert one.plan()["fused_step"] == int(one.plan()["num_splits"] == 1)
    assert check_step_against_oracle(w, one, range(w.batch)) <= max(1, w.batch * w.spec.num_kv_heads // 20)


@pytest.mark.parametrize("name", ["gqa_bf16", "largebatch_bf16", "longgen_bf16"])
def test_full_size_bf16_centroid_step_equals_calls(name):
    """The benchmarked shapes with bf16-copy scoring: whole step equals the
    separate calls bit for bit; sampled sequences match the oracle."""
    sp = W.spec(name, headroom_tokens=max(64, W.spec(name).headroom_tokens))
    w = W.make(sp, "cuda", seed=2)
    one = step_vs_calls(w, score_bf16=True)
    assert one.plan()["fused_step"] == 1
    assert check_step_against_oracle(w, one, [0, w.batch // 2, w.batch - 1]) <= 1
    del w, one
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,batch,lengths", [("largebatch_bf16", 40, ("uniform", 2000, 9000)),
                                                ("longgen_bf16", 48, ("uniform", 8200, 12000))])
def test_paired_rows_decode_step(name, batch, lengths):
    """Between one and two rounds of 8-wave whole-step blocks (320 and 384
    segments on 256 compute units) the step kernel ranks the sequences
    itself and pairs rows of long sequences with rows of short ones: the same
    bits as the separate calls, and the oracle's results on a sample."""
    sp = W.spec(name, batch=batch, lengths=lengths, headroom_tokens=40)
    w = W.make(sp, "cuda", seed=21)
    one = step_vs_calls(w, appends=2)
    plan = one.plan()
    assert plan["fused_step"] == 1
    segs = batch * sp.num_kv_heads
    if plan["num_cus"] < segs <= 2 * plan["num_cus"] and plan["num_cus"] % sp.num_kv_heads == 0:
        assert plan["pair_segments"] == plan["num_cus"] // sp.num_kv_heads
    assert check_step_against_oracle(w, one, [0, batch // 2, batch - 1]) <= 1
    del w, one
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gqa_small", "large_small", "longgen_small"])
def test_fused_decode_step_matches_oracle(name):
    """One split per segment (the whole-step kernel where the shape allows),
    after appends, against the oracle for every sequence."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=20), "cpu", seed=16))
    step = DecodeStep(w, num_splits=1)
    step.rebuild_centroids()
    for _ in range(3):
        w.append_token()
        step.run()
    T.sync()
    differing = check_step_against_oracle(w, step, range(w.batch))
    assert differing <= max(1, w.batch * w.spec.num_kv_heads // 20)


@pytest.mark.parametrize("name", ["mla_small", "mla16_small"])
def test_mla_latent_only_scoring(name):
    """The rope-unaware MLA indexer (score on the 512 latent columns):
    oracle parity for every sequence, and the whole-step call equals the
    separate calls bit for bit."""
    from test_gpu_parity import pipeline_check
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=20), "cpu", seed=17))
    _, _, differing = pipeline_check(w, range(w.batch), DecodeStep(w, score_dim=512))
    assert differing <= max(1, w.batch // 20)
    step_vs_calls(w, score_dim=512)


@pytest.mark.parametrize("k,n_sink,n_local", [(0, 1, 1), (3, 0, 0), (200, 1, 1), (5, 2, 0),
                                              (5, 0, 3)])
@pytest.mark.parametrize("name", ["gqa_small", "mla_small", "mla16_small"])
def test_step_selection_budgets(name, k, n_sink, n_local):
    """The whole-step kernels select inside the attention kernel: other
    budgets and forced windows (none, k = 0, k beyond the page count) give
    the same bits as the separate calls, and the oracle's attention."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=20), "cpu", seed=23))
    one = step_vs_calls(w, appends=1, k=k, n_sink=n_sink, n_local=n_local)
    assert check_step_against_oracle(w, one, range(w.batch)) <= max(1, w.batch // 20)


@pytest.mark.parametrize("indexer", ["centroid", "bounds"])
def test_selection_beyond_one_split(indexer):
    """More than 256 selected pages per segment (k = 300): the plan needs two
    or more attention splits, so the step runs as separate kernels with the
    split merge; same bits as the separate calls, and the oracle."""
    sp = W.spec("gqa_bf16", batch=2, num_q_heads=4, num_kv_heads=2,
                lengths=("list", (6000, 9000)), headroom_tokens=16)
    w = W.make(sp, "cuda", seed=24)
    kw = dict(k=300, n_sink=1, n_local=1)
    if indexer == "bounds":
        from test_gpu_bounds import bound_step_vs_calls, check_against_oracle as check_bounds_step
        one = bound_step_vs_calls(w, appends=1, **kw)
        assert one.plan()["num_splits"] >= 2 and one.plan()["fused_step"] == 0
        assert check_bounds_step(w, one, range(2)) == 0
    else:
        one = step_vs_calls(w, appends=1, **kw)
        assert one.plan()["num_splits"] >= 2 and one.plan()["fused_step"] == 0
        assert check_step_against_oracle(w, one, range(2)) == 0
    del w, one
    torch.cuda.empty_cache()


def test_mla_selection_beyond_one_split():
    """MLA with more than 256 selected pages per sequence: the select +
    attention kernel runs several splits of one selection and the merge; same
    bits as the separate calls, and the oracle."""
    sp = W.spec("mla_bf16", batch=2, lengths=("list", (20000, 30000)), headroom_tokens=64)
    w = W.make(sp, "cuda", seed=25)
    one = step_vs_calls(w, appends=1, k=300, n_sink=1, n_local=1)
    assert one.plan()["num_splits"] >= 2
    assert check_step_against_oracle(w, one, range(2)) == 0
    del w, one
    torch.cuda.empty_cache()
