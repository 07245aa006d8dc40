"""GPU radix top-k against the oracle on identical fp32 scores (bit-exact).

Scores are fed to the kernel directly, so both sides rank the same fp32
values: the exact mode must return exactly the oracle's pages, and the
approximate mode exactly the oracle's reading of it (same remap, same
boundary bucket, same random window).
"""

import numpy as np
import pytest
import torch

from oracle import vx_oracle as O
from sparse_attention_decode_amd import binding as V

pytestmark = pytest.mark.gpu

P = 16


def segments(seed, batch, hkv, max_n):
    rng = np.random.default_rng(seed)
    ns = rng.integers(1, max_n + 1, size=batch)
    ns[0] = 1
    if batch > 2:
        ns[1] = max_n
    scores = []
    for b in range(batch):
        for g in range(hkv):
            kind = (b * hkv + g) % 5
            n = ns[b]
            if kind == 0:
                s = rng.standard_normal(n)
            elif kind == 1:
                s = rng.integers(-3, 4, size=n).astype(np.float64)  # heavy ties
            elif kind == 2:
                s = np.zeros(n)
                s[rng.random(n) < 0.5] = -0.0
            elif kind == 3:
                s = rng.standard_normal(n) * 1e-30  # tiny magnitudes, denormal-free
            else:
                s = np.round(rng.standard_normal(n), 2) * 1000.0
            scores.append(s.astype(np.float32))
    return ns, scores


def run_topk(ns, scores, hkv, k, n_sink, n_local, mode, rnd):
    batch = len(ns)
    indptr = np.zeros(batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(ns)
    nnz = int(indptr[-1])
    sc = np.zeros((hkv, nnz), dtype=np.float32)
    for b in range(batch):
        for g in range(hkv):
            sc[g, indptr[b]:indptr[b + 1]] = scores[b * hkv + g]
    dev = torch.device("cuda")
    d_indptr = torch.from_numpy(indptr).to(dev)
    d_lens = torch.from_numpy((ns * P).astype(np.int32)).to(dev)
    d_ids = torch.arange(nnz, dtype=torch.int32, device=dev)
    pages = V.make_pages(batch, P, nnz, nnz, int(ns.max()), d_indptr, d_ids, d_lens)
    stride = max(1, k + n_sink + n_local)
    sel = torch.full((batch, hkv, stride), -7, dtype=torch.int32, device=dev)
    cnt = torch.zeros((batch, hkv), dtype=torch.int32, device=dev)
    d_sc = torch.from_numpy(sc).to(dev)
    d_rnd = torch.from_numpy(rnd.view(np.int32)).to(dev)
    V.vx_topk_pages(pages, hkv, d_sc, k, n_sink, n_local, mode, d_rnd, sel, stride, cnt)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("k,n_sink,n_local", [(16, 1, 1), (8, 0, 1), (128, 1, 2), (64, 0, 0),
                                              (0, 1, 1), (1, 0, 0), (5, 3, 3), (96, 2, 2)])
@pytest.mark.parametrize("mode", [V.VX_TOPK_EXACT, V.VX_TOPK_APPROX])
@pytest.mark.parametrize("max_n", [250, 2100])
def test_topk_bit_exact(k, n_sink, n_local, mode, max_n):
    """max_n 250: one wave per segment (register select); 2100: one block per
    segment (local top-k per wave then one wave over the candidates for
    k <= 96, digit passes for k = 128)."""
    hkv, batch = 3, 9
    ns, scores = segments(1000 + k + max_n, batch, hkv, max_n=max_n)
    rnd = np.random.default_rng(k).integers(0, 2**32, size=(batch, hkv), dtype=np.uint64).astype(np.uint32)
    sel, cnt = run_topk(ns, scores, hkv, k, n_sink, n_local, mode, rnd)
    for b in range(batch):
        for g in range(hkv):
            s = scores[b * hkv + g]
            if mode == V.VX_TOPK_EXACT:
                want = O.topk_exact(s.astype(np.float64), k, n_sink, n_local)
            else:
                want = O.topk_approx(s, k, n_sink, n_local, int(rnd[b, g]))
            stride = max(1, k + n_sink + n_local)
            full = np.full(stride, -1)
            full[:len(want)] = want
            np.testing.assert_array_equal(sel[b, g], full, err_msg=f"b={b} g={g} n={ns[b]}")
            assert cnt[b, g] == int((want >= 0).sum())


@pytest.mark.parametrize("ns", [(5000, 3, 4100), (4000, 3, 2900)])
def test_topk_large_segments(ns):
    """Long segments (one block per segment) next to a 3-page one; up to 4096
    pages the waves' ranges fit their registers (local top-k then one wave
    over the candidates), beyond that the digit passes run."""
    hkv, batch = 2, 3
    rng = np.random.default_rng(5)
    ns = np.array(ns)
    scores = [rng.standard_normal(ns[b]).astype(np.float32) for b in range(batch) for _ in range(hkv)]
    rnd = np.zeros((batch, hkv), dtype=np.uint32)
    sel, cnt = run_topk(ns, scores, hkv, 64, 1, 1, V.VX_TOPK_EXACT, rnd)
    for b in range(batch):
        for g in range(hkv):
            want = O.topk_exact(scores[b * hkv + g].astype(np.float64), 64, 1, 1)
            np.testing.assert_array_equal(sel[b, g][:len(want)], want)


@pytest.mark.parametrize("mode", [V.VX_TOPK_EXACT, V.VX_TOPK_APPROX])
def test_topk_maximum_segment(mode):
    """A segment at the largest supported page count (16000: its keys and
    histograms take more than 64 KB of LDS) next to a short one; exact mode
    against the oracle, approximate mode against the oracle's reading of it."""
    hkv, batch = 1, 2
    rng = np.random.default_rng(9)
    ns = np.array([16000, 40])
    scores = [rng.standard_normal(n).astype(np.float32) for n in ns]
    rnd = rng.integers(0, 2**32, size=(batch, hkv), dtype=np.uint64).astype(np.uint32)
    sel, cnt = run_topk(ns, scores, hkv, 200, 1, 2, mode, rnd)
    for b in range(batch):
        s64 = scores[b].astype(np.float64)
        if mode == V.VX_TOPK_EXACT:
            want = O.topk_exact(s64, 200, 1, 2)
        else:
            want = O.topk_approx(scores[b], 200, 1, 2, int(rnd[b, 0]))
        np.testing.assert_array_equal(sel[b, 0][:len(want)], want)  # padded with -1
        assert cnt[b, 0] == int((want >= 0).sum())


@pytest.mark.parametrize("case", ["few_survivors", "many_survivors", "tied_fallback",
                                  "short_ranges_fallback"])
def test_topk_block_bound_cases(case):
    """Segments of more than 256 pages go to the block select, whose exact
    path first bounds the k-th largest key from below by each wave's
    ceil(k / waves) largest keys and selects among the keys at or above the
    bound. Cases: distinct scores with a small k (few survivors) and a larger
    k (up to 256 survivors); scores from 5 values (more than 256 keys tie at
    the bound: the select falls back to its other paths); a sink long enough
    to leave the first wave's range without candidates, so the ranges' keys
    do not reach k (fallback as well). Each against the oracle, bit-exact."""
    rng = np.random.default_rng(77)
    hkv = 1
    if case == "few_survivors":
        ns, k, n_sink, n_local = np.array([1024, 700]), 32, 1, 1
        scores = [rng.standard_normal(n).astype(np.float32) for n in ns]
    elif case == "many_survivors":
        ns, k, n_sink, n_local = np.array([1024, 2048]), 64, 1, 1
        scores = [rng.standard_normal(n).astype(np.float32) for n in ns]
    elif case == "tied_fallback":
        ns, k, n_sink, n_local = np.array([1024, 600]), 32, 1, 1
        scores = [rng.integers(0, 5, size=n).astype(np.float32) for n in ns]
    else:
        ns, k, n_sink, n_local = np.array([270, 300]), 64, 40, 1
        scores = [rng.standard_normal(n).astype(np.float32) for n in ns]
    rnd = np.zeros((len(ns), hkv), dtype=np.uint32)
    sel, cnt = run_topk(ns, scores, hkv, k, n_sink, n_local, V.VX_TOPK_EXACT, rnd)
    for b in range(len(ns)):
        want = O.topk_exact(scores[b].astype(np.float64), k, n_sink, n_local)
        np.testing.assert_array_equal(sel[b, 0][:len(want)], want, err_msg=f"{case} b={b}")
        assert (sel[b, 0][len(want):] == -1).all()
        assert cnt[b, 0] == len(want)
