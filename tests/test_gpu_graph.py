"""The step captured in a HIP graph (as bench.py times it) and replayed
several times, with eager work on the same buffers between replays, gives the
eager call's bits every time."""

import pytest
import torch

import vx_testlib as T
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def snapshot(step):
    return [t.clone() for t in (step.out, step.lse, step.sel, step.sel_count, step.scores)]


@pytest.mark.parametrize("name,indexer,fused", [
    ("gqa_small", "centroid", True), ("gqa_small", "centroid", False),
    ("mla_small", "centroid", True), ("longgen_small", "bounds", True),
    ("large_small", "bounds", False), ("tiny_fp32", "centroid", True)])
def test_graph_replay_matches_eager(name, indexer, fused):
    w = on_gpu(W.make(SMALL[name].replace(headroom_tokens=8), "cpu", seed=50))
    step = DecodeStep(w, indexer=indexer, fused=fused)
    step.rebuild()
    w.append_token()
    step.run()
    T.sync()
    want = snapshot(step)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step.run()
    T.sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream, capture_error_mode="thread_local"):
        step.run()
    T.sync()
    for i in range(4):
        step.out.fill_(float(i + 1))
        step.sel.fill_(-7)
        step.sel_count.fill_(99)
        step.run()  # eager work on the same buffers between replays
        T.sync()
        step.out.fill_(0.0)
        with torch.cuda.stream(stream):
            g.replay()
        T.sync()
        got = snapshot(step)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {i}"
