"""Host checks of the seeded input generators (no GPU)."""
import math

import numpy as np
import pytest
import torch

from sparse_attention_decode_amd import workloads as W
from oracle import vx_oracle as O

SMALL = {
    "tiny_fp32": {},
    "gqa_bf16": dict(batch=3, lengths=("uniform", 100, 300)),
    "longgen_bf16": dict(batch=3, lengths=("uniform", 200, 500), headroom_tokens=40),
    "mla_bf16": dict(batch=2, lengths=("uniform", 300, 700)),
    "largebatch_bf16": dict(batch=4, lengths=("lognormal", 400, math.log(2.0), 100, 1600)),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_page_tables_are_consistent(name):
    w = W.make(W.spec(name, **SMALL[name]), "cpu", seed=0)
    s = w.spec
    assert w.indptr[0] == 0 and np.all(np.diff(w.indptr) >= 1)
    assert len(set(w.page_ids.tolist())) == w.nnz  # no page shared
    assert w.page_ids.min() >= 0 and w.page_ids.max() < w.pool_pages
    P = s.page_size
    for b in range(s.batch):
        assert 1 <= w.seq_lens[b] <= (w.indptr[b + 1] - w.indptr[b]) * P
    assert w.k_pool.shape == (w.pool_pages, s.num_kv_heads, P, s.head_dim_k)
    assert (w.v_pool is None) == s.mla
    assert w.q.shape == (s.batch, s.num_q_heads, s.head_dim_k)
    if name == "tiny_fp32":
        assert w.pool_pages == 128 and w.nnz == 64 and int(w.seq_lens[0]) == 1024


def test_seeded_and_reproducible():
    a = W.make(W.spec("gqa_bf16", **SMALL["gqa_bf16"]), "cpu", seed=0)
    b = W.make(W.spec("gqa_bf16", **SMALL["gqa_bf16"]), "cpu", seed=0)
    c = W.make(W.spec("gqa_bf16", **SMALL["gqa_bf16"]), "cpu", seed=1)
    assert torch.equal(a.k_pool, b.k_pool) and np.array_equal(a.page_ids, b.page_ids)
    assert not torch.equal(a.k_pool, c.k_pool)


def test_boost_recipe_five_percent_along_one_direction():
    """5% of token positions per sequence get +3 along one unit direction per
    KV head: the mean key is ~0.15 u, and projecting on it splits off ~5%."""
    w = W.make(W.spec("gqa_bf16", batch=16, lengths=("uniform", 4096, 4096)), "cpu")
    s = w.spec
    for g in range(s.num_kv_heads):
        rows = []
        for b in range(s.batch):
            lo, hi = int(w.indptr[b]), int(w.indptr[b + 1])
            ids = torch.from_numpy(w.page_ids[lo:hi].astype(np.int64))
            rows.append(w.k_pool[ids, g].float().reshape(-1, s.head_dim_k)[: int(w.seq_lens[b])])
        keys = torch.cat(rows)
        mean = keys.mean(0)
        assert 0.11 < mean.norm().item() < 0.19
        proj = keys @ (mean / mean.norm())
        frac = (proj > 2.0).float().mean().item()
        assert 0.05 < frac < 0.09


def test_random_walk_drift_and_append():
    sp = W.spec("longgen_bf16", batch=2, lengths=("uniform", 1600, 1600), headroom_tokens=32)
    w = W.make(sp, "cpu")
    seq = w.host_sequence(0)
    cent = O.centroids(seq["k"], seq["seq_len"], sp.page_size)
    # neighbouring page means are close (walk step 0.1), far pages drift apart
    near = np.abs(cent[1:] - cent[:-1]).mean()
    far = np.abs(cent[-1] - cent[0]).mean()
    assert far > 2 * near
    L0 = int(w.seq_lens[0])
    for _ in range(32):
        w.append_token()
    assert int(w.seq_lens[0]) == L0 + 32
    with pytest.raises(ValueError):
        for _ in range(64):
            w.append_token()


def test_mla_column_scales():
    w = W.make(W.spec("mla_bf16", **SMALL["mla_bf16"]), "cpu")
    k = w.k_pool.float()
    lat, rope = k[..., :512].std().item(), k[..., 512:].std().item()
    assert abs(lat - 0.5) < 0.02 and abs(rope - 1.0) < 0.04
