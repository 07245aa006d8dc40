"""vx_decode_step_static (no workspace argument; the split partials live in
the library's own device scratch) against vx_decode_step with a caller
workspace: the same kernels, so the same bits, on two calls in a row, the
second on a smaller input; and a step whose partials exceed the scratch is
refused before any launch."""

import numpy as np
import pytest
import torch

from sparse_attention_decode_amd import binding as V
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep

pytestmark = pytest.mark.gpu


def both(w, num_splits=0):
    """One step through vx_decode_step (workspace from torch) and one through
    vx_decode_step_static, each on its own centroid copy and outputs."""
    a = DecodeStep(w, num_splits=num_splits)
    b = DecodeStep(w, num_splits=num_splits)
    a.rebuild()
    b.rebuild()
    a.step()
    V.vx_decode_step_static(b.pages, b.geom, w.q, w.k_pool, w.v_pool, b.centroids, b.cent_bf16,
                            True, b.score_scale, b.sm_scale, b.k, b.n_sink, b.n_local, b.mode,
                            w.d_rand_u32, b.scores, b.sel, b.k_out, b.sel_count, b.out, b.lse,
                            num_splits)
    torch.cuda.synchronize()
    return a, b


def assert_same(a, b, tag):
    assert a.plan()["num_splits"] > 1 or a.num_splits > 1, f"{tag}: not a split step"
    for name in ("out", "lse", "sel", "sel_count", "scores", "centroids"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x, y), f"{tag}: {name} differs"


@pytest.mark.parametrize("name,big,small", [
    ("mla_bf16", dict(batch=4, lengths=("list", (20000, 9000, 31000, 4100))),
     dict(batch=2, lengths=("list", (5000, 700)))),
    ("gqa_bf16", dict(batch=3, lengths=("list", (3000, 900, 2500))),
     dict(batch=2, lengths=("list", (400, 1700)))),
])
def test_static_scratch_matches_workspace(name, big, small):
    splits = 0 if name == "mla_bf16" else 3  # GQA: force a split step
    for tag, kw in (("first", big), ("second, smaller", small)):
        w = W.make(W.spec(name, **kw), "cuda", seed=7)
        a, b = both(w, splits)
        assert_same(a, b, f"{name} {tag}")


def test_static_scratch_limit():
    """Partials above the scratch size: VX_ERR_WORKSPACE, nothing launched
    (the pointers are never dereferenced)."""
    bad = 0x1000
    pages = V.make_pages(16, 16, 4000, 3200, 200, bad, bad, bad)
    geom = V.make_geom(32, 8, 128, 128, 0, V.VX_BF16, V.VX_BF16)
    with pytest.raises(V.VxError) as e:
        V.vx_decode_step_static(pages, geom, bad, bad, bad, bad, None, True, 0.1, 0.1, 128, 1, 2,
                                V.VX_TOPK_EXACT, None, bad, bad, 131, bad, bad, bad, 130)
    assert e.value.status == V.VX_ERR_WORKSPACE, e.value
    assert "static scratch" in str(e.value)


def static_call(b, w, num_splits):
    V.vx_decode_step_static(b.pages, b.geom, w.q, w.k_pool, w.v_pool, b.centroids, b.cent_bf16,
                            True, b.score_scale, b.sm_scale, b.k, b.n_sink, b.n_local, b.mode,
                            w.d_rand_u32, b.scores, b.sel, b.k_out, b.sel_count, b.out, b.lse,
                            num_splits, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("name,kw,splits", [
    ("mla_bf16", dict(batch=3, lengths=("list", (20000, 9000, 4100))), 0),
    ("gqa_bf16", dict(batch=3, lengths=("list", (3000, 900, 2500))), 3),
])
def test_static_step_under_graph_capture(name, kw, splits):
    """The call the entry point exists for: captured in a HIP graph (no
    allocation inside the capture), replayed four times with eager work on
    the same buffers between replays; every replay gives vx_decode_step's
    bits."""
    w = W.make(W.spec(name, **kw), "cuda", seed=11)
    a, b = both(w, splits)  # eager: the address lookup happens here, outside the capture
    assert_same(a, b, f"{name} eager")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream, capture_error_mode="thread_local"):
        static_call(b, w, splits)
    torch.cuda.synchronize()
    for i in range(4):
        b.out.fill_(float(i + 1))
        b.sel.fill_(-7)
        b.lse.fill_(0.5)
        static_call(b, w, splits)  # eager use of the same scratch between replays
        torch.cuda.synchronize()
        b.out.fill_(0.0)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert_same(a, b, f"{name} replay {i}")
