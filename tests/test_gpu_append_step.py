"""vx_append_decode_step against its two calls: vx_centroid_update with the
new token's K/V rows (first_token = -1), then vx_decode_step without the
refresh. Bit for bit on the pools, the centroids, the scores, the selection
and the attention, on the one-kernel GQA step (matrix-core and vector
bodies), the split paths (the append kernel first) and MLA."""

import numpy as np
import pytest
import torch

import vx_testlib as T
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu
from test_gpu_index import used_pages, valid_entries
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def append_vs_calls(w1, appends, num_splits=0):
    w2 = w1.replicate()
    one = DecodeStep(w1, num_splits=num_splits)
    two = DecodeStep(w2, num_splits=num_splits)
    one.rebuild_centroids()
    two.rebuild_centroids()
    used = used_pages(w1)
    for _ in range(appends):
        w1.append_token()
        w2.append_token()
        one.run_append(one_call=True)
        two.run_append(one_call=False)
        T.sync()
        valid = valid_entries(w1)
        assert torch.equal(w1.k_pool, w2.k_pool)
        if w1.v_pool is not None:
            assert torch.equal(w1.v_pool, w2.v_pool)
        assert torch.equal(one.centroids[used], two.centroids[used])
        if one.cent_bf16 is not None:
            assert torch.equal(one.cent_bf16[used], two.cent_bf16[used])
        assert torch.equal(one.scores[:, valid], two.scores[:, valid])
        assert torch.equal(one.sel_count, two.sel_count)
        assert torch.equal(one.sel, two.sel)
        assert torch.equal(one.out, two.out)
        assert torch.equal(one.lse, two.lse)
    return one


@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("name", ["tiny_fp32", "gqa_small", "longgen_small", "large_small",
                                  "mla_small"])
def test_append_step_equals_calls(name, num_splits):
    """Three appends (lengths crossing page boundaries on the way); one split
    per segment takes the one-kernel GQA step, which writes the rows itself."""
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=31))
    one = append_vs_calls(w, 3, num_splits)
    s = w.spec
    fused = one.plan()["num_splits"] == 1 and not s.mla and one.k_out <= 256
    assert one.plan()["fused_step"] == int(fused)


def test_append_step_writes_the_new_rows():
    """After the one-call append step, the newest token's slot holds k_new /
    v_new, and its page's centroid equals a rebuild over the written pool."""
    sp = W.spec("longgen_bf16", batch=3, lengths=("list", (500, 511, 512)), headroom_tokens=32)
    w = on_gpu(W.make(sp, "cpu", seed=10))
    step = DecodeStep(w, num_splits=1)
    assert step.plan()["fused_step"] == 1
    step.rebuild_centroids()
    w.append_token()
    step.run_append(one_call=True)
    T.sync()
    s = w.spec
    for b in range(s.batch):
        t = int(w.seq_lens[b]) - 1
        pid = int(w.page_ids[w.indptr[b] + t // s.page_size])
        assert torch.equal(w.k_pool[pid, :, t % s.page_size], step.k_new[b])
        assert torch.equal(w.v_pool[pid, :, t % s.page_size], step.v_new[b])
    inc = step.centroids.clone()
    step.rebuild_centroids()
    T.sync()
    used = used_pages(w)
    assert torch.equal(inc[used], step.centroids[used])


@pytest.mark.parametrize("name", ["longgen_bf16", "mla_bf16"])
def test_full_size_append_step_equals_calls(name):
    """The timed appending step at full size: the one-kernel step (long
    generation) and MLA's append kernel + scorer + select/attention + merge."""
    sp = W.spec(name, headroom_tokens=max(64, W.spec(name).headroom_tokens))
    w = W.make(sp, "cuda", seed=4)
    one = append_vs_calls(w, 2)
    assert one.plan()["fused_step"] == (0 if sp.mla else 1)
    del w, one
    torch.cuda.empty_cache()
