"""GPU parity of the whole step against the CPU oracle on seeded inputs.

Small variants of each workload span several tiles and ragged tails and are
checked on every sequence; the full-size workloads run in the launch
configuration the benchmark times and are checked on sampled sequences
(the oracle regenerates nothing: it reads host copies of the same inputs).
"""

import math

import numpy as np
import pytest
import torch

import vx_testlib as T
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_fp32": W.spec("tiny_fp32"),
    "gqa_small": W.spec("gqa_bf16", batch=5, lengths=("uniform", 100, 700)),
    "longgen_small": W.spec("longgen_bf16", batch=4, lengths=("uniform", 1000, 3000),
                            headroom_tokens=40),
    "large_small": W.spec("largebatch_bf16", batch=6,
                          lengths=("lognormal", 4000, math.log(2.0), 1000, 16000)),
    "mla_small": W.spec("mla_bf16", batch=4, lengths=("uniform", 2000, 6000)),
    "mla16_small": W.spec("mla_bf16", batch=3, num_q_heads=16, lengths=("uniform", 1500, 5000)),
}


def pipeline_check(w, sample, step=None):
    step = step or DecodeStep(w)
    step.rebuild_centroids()
    step.score()
    step.select()
    step.attend()
    T.sync()
    refs = {b: T.oracle_seq(w, step, b) for b in sample}
    out = step.out.cpu().double().numpy()
    lse = step.lse.cpu().double().numpy()
    G = w.spec.num_q_heads // w.spec.num_kv_heads
    differing = 0
    for b, r in refs.items():
        T.check_centroids(w, step, b, r)
        T.check_scores(w, step, b, r)
        same = T.check_selection(w, step, b, r)
        for g, ok in enumerate(same):
            if ok:
                T.check_attention(w, out[b], lse[b], r["out"], r["lse"],
                                  heads=range(g * G, (g + 1) * G), tag=f"b={b} g={g}")
            else:
                differing += 1
                T.check_attention_on_gpu_selection(w, step, b, r, out[b], lse[b], g,
                                                   tag=f"b={b} g={g}")
    # attention on exactly the oracle's selection, every head
    sel, cnt = T.sel_tensor_from_oracle(w, step, refs)
    step.attend(sel=sel, sel_count=cnt)
    T.sync()
    out = step.out.cpu().double().numpy()
    lse = step.lse.cpu().double().numpy()
    for b, r in refs.items():
        T.check_attention(w, out[b], lse[b], r["out"], r["lse"], tag=f"b={b} oracle sel")
    return step, refs, differing


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads_every_sequence(name):
    w = W.make(SMALL[name], "cpu", seed=0)
    w = W.Workload(spec=w.spec, device=torch.device("cuda"), seq_lens=w.seq_lens,
                   indptr=w.indptr, page_ids=w.page_ids, pool_pages=w.pool_pages,
                   q=w.q.cuda(), k_pool=w.k_pool.cuda(),
                   v_pool=None if w.v_pool is None else w.v_pool.cuda(), rand_u32=w.rand_u32)
    _, _, differing = pipeline_check(w, range(w.batch))
    assert differing <= max(1, w.batch * w.spec.num_kv_heads // 20)


@pytest.mark.parametrize("name,sample", [
    ("tiny_fp32", [0]),
    ("gqa_bf16", list(range(32))),
    ("longgen_bf16", [0, 17, 63]),
    ("largebatch_bf16", [0, 100, 255]),
    ("mla_bf16", [0, 13, 31]),
])
def test_full_size_workloads_sampled(name, sample):
    w = W.make(W.spec(name), "cuda", seed=0)
    _, _, differing = pipeline_check(w, sample)
    assert differing <= max(1, len(sample) * w.spec.num_kv_heads // 20)
    del w
    torch.cuda.empty_cache()


def test_full_size_approximate_selection_on_gpu_scores():
    """The large-batch workload in approximate top-k mode, at full size in the
    benchmarked launch (one kernel per step): for sampled sequences, every KV
    head's selection equals the oracle's approximate selection run on the
    GPU's own fp32 scores, bit for bit (the same remap, boundary bucket and
    random window)."""
    from oracle import vx_oracle as O
    from sparse_attention_decode_amd import binding as V
    s = W.spec("largebatch_bf16")
    w = W.make(s, "cuda", seed=0)
    step = DecodeStep(w, mode=V.VX_TOPK_APPROX)
    step.rebuild()
    step.run()
    T.sync()
    assert step.plan()["fused_step"]
    scores = step.scores.cpu().numpy()
    sel = step.sel.cpu().numpy()
    cnt = step.sel_count.cpu().numpy()
    for b in (0, 37, 100, 181, 255):
        lo, n = int(w.indptr[b]), w.n_pages(b)
        for g in range(s.num_kv_heads):
            want = O.topk_approx(scores[g, lo:lo + n], step.k, step.n_sink, step.n_local,
                                 int(w.rand_u32[b, g]))
            full = np.full(step.k_out, -1)
            full[:len(want)] = want
            np.testing.assert_array_equal(sel[b, g], full, err_msg=f"b={b} g={g} n={n}")
            assert cnt[b, g] == int((want >= 0).sum())
    del w, step
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,sample", [("gqa_small", None), ("large_small", None),
                                         ("gqa_bf16", [0, 9, 20, 31]),
                                         ("longgen_bf16", [0, 40, 63])])
def test_bf16_centroid_scoring(name, sample):
    """GQA scores on the centroids' bf16 copy (vx_page_scores on the copy,
    the separate calls): scores within the condition-aware bound of the
    oracle's reading (bf16 rounding of the fp32 token-order centroid), the
    selection, and the attention, as in the default pipeline."""
    if sample is None:
        w = W.make(SMALL[name], "cpu", seed=3)
        w = W.Workload(spec=w.spec, device=torch.device("cuda"), seq_lens=w.seq_lens,
                       indptr=w.indptr, page_ids=w.page_ids, pool_pages=w.pool_pages,
                       q=w.q.cuda(), k_pool=w.k_pool.cuda(), v_pool=w.v_pool.cuda(),
                       rand_u32=w.rand_u32)
        sample = range(w.batch)
    else:
        w = W.make(W.spec(name), "cuda", seed=3)
    step = DecodeStep(w, score_bf16=True)
    assert step.cent_bf16 is not None
    _, _, differing = pipeline_check(w, sample, step=step)
    assert differing <= max(1, len(sample) * w.spec.num_kv_heads // 20)
    del w, step
    torch.cuda.empty_cache()
