"""The cache stage bit for bit: the GPU's centroids (full rebuild, the
stand-alone refresh, and the refresh inside the indexer and whole-step
kernels, over appends that cross page boundaries) equal the oracle's fp32
definition exactly (token-order fp32 sum, one IEEE division), and MLA's bf16
copy equals its round-to-nearest-even."""

import numpy as np
import pytest
import torch

import vx_testlib as T
from oracle import vx_oracle as O
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def check_exact(w, step):
    P = w.spec.page_size
    for b in range(w.batch):
        seq = w.host_sequence(b)
        c32 = O.centroids_fp32(seq["k"], seq["seq_len"], P)
        n = c32.shape[0]
        if n == 0:
            continue
        got = T.gpu_centroids(w, step, b, n)
        np.testing.assert_array_equal(got, c32.astype(np.float64), err_msg=f"b={b}")
        if w.spec.mla:
            lo = int(w.indptr[b])
            ids = torch.from_numpy(w.page_ids[lo:lo + n].astype(np.int64)).to(w.device)
            shadow = step.cent_bf16.index_select(0, ids).double().cpu().numpy()
            np.testing.assert_array_equal(shadow, O.round_to_bf16(c32.astype(np.float64)),
                                          err_msg=f"bf16 b={b}")


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", list(SMALL))
def test_centroids_bit_exact(name, fused):
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=40), "cpu", seed=41))
    step = DecodeStep(w, fused=fused)
    step.rebuild_centroids()
    T.sync()
    check_exact(w, step)
    for _ in range(20):  # crosses a page boundary at P = 16
        w.append_token()
        step.run()
    T.sync()
    check_exact(w, step)
