"""With a budget of every page, the sparse step is full attention: the GPU
selection must be every page in use, and the output must equal softmax
attention over the whole contiguous sequence, computed here directly in
numpy fp64 (not through the oracle module)."""

import numpy as np
import pytest
import torch

import vx_testlib as T
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu

pytestmark = pytest.mark.gpu


def dense_reference(w, b, sm_scale):
    """out [Hq][Dv], lse [Hq] of full softmax attention for sequence b."""
    s = w.spec
    seq = w.host_sequence(b)
    L = seq["seq_len"]
    k = seq["k"].transpose(0, 2, 1, 3).reshape(-1, s.num_kv_heads, s.head_dim_k)[:L]
    v = k[..., :s.head_dim_v] if s.mla else \
        seq["v"].transpose(0, 2, 1, 3).reshape(-1, s.num_kv_heads, s.head_dim_v)[:L]
    G = s.num_q_heads // s.num_kv_heads
    out = np.zeros((s.num_q_heads, s.head_dim_v))
    lse = np.zeros(s.num_q_heads)
    for h in range(s.num_q_heads):
        g = h // G
        z = sm_scale * (k[:, g, :] @ seq["q"][h])
        mx = z.max()
        e = np.exp(z - mx)
        out[h] = (e @ v[:, g, :]) / e.sum()
        lse[h] = mx + np.log(e.sum())
    return out, lse


CASES = {
    "tiny_fp32": W.spec("tiny_fp32", lengths=("fixed", 700)),
    "gqa": W.spec("gqa_bf16", batch=3, lengths=("list", (150, 900, 1500))),
    "large": W.spec("largebatch_bf16", batch=2, lengths=("list", (3000, 5100))),
    "mla": W.spec("mla_bf16", batch=2, lengths=("list", (2500, 4000))),
}


@pytest.mark.parametrize("num_splits", [0, 1])
@pytest.mark.parametrize("name", list(CASES))
def test_every_page_selected_is_full_attention(name, num_splits):
    w = on_gpu(W.make(CASES[name], "cpu", seed=21))
    step = DecodeStep(w, k=w.max_pages, n_sink=0, n_local=0, num_splits=num_splits)
    step.rebuild_centroids()
    step.run()
    T.sync()
    sel, cnt = step.sel.cpu().numpy(), step.sel_count.cpu().numpy()
    out, lse = step.out.cpu().double().numpy(), step.lse.cpu().double().numpy()
    for b in range(w.batch):
        n = w.n_pages(b)
        for g in range(w.spec.num_kv_heads):
            assert cnt[b, g] == n
            assert list(sel[b, g, :n]) == list(range(n))
            assert (sel[b, g, n:] == -1).all()
        ref_out, ref_lse = dense_reference(w, b, step.sm_scale)
        T.check_attention(w, out[b], lse[b], ref_out, ref_lse, tag=f"{name} b={b}")
