"""GPU edge cases, launch-shape invariance, determinism and the cache stage's
incremental update."""

import numpy as np
import pytest
import torch

import vx_testlib as T
from oracle import vx_oracle as O
from sparse_attention_decode_amd import binding as V
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_parity import pipeline_check

pytestmark = pytest.mark.gpu


def on_gpu(w: W.Workload) -> W.Workload:
    return W.Workload(spec=w.spec, device=torch.device("cuda"), seq_lens=w.seq_lens,
                      indptr=w.indptr, page_ids=w.page_ids, pool_pages=w.pool_pages,
                      q=w.q.cuda(), k_pool=w.k_pool.cuda(),
                      v_pool=None if w.v_pool is None else w.v_pool.cuda(), rand_u32=w.rand_u32)


EDGE_LENS = (1, 16, 17, 33, 48, 160, 300, 1)


@pytest.mark.parametrize("base", ["gqa_bf16", "tiny_fp32", "largebatch_bf16", "mla_bf16"])
def test_short_and_partial_sequences(base):
    """seq_len 1, exact page multiples, one token into a new page, fewer
    pages than k + forced (everything selected)."""
    sp = W.spec(base, batch=len(EDGE_LENS), lengths=("list", EDGE_LENS), topk=4,
                pool=("factor", 1.5))
    pipeline_check(on_gpu(W.make(sp, "cpu", seed=3)), range(len(EDGE_LENS)))


@pytest.mark.parametrize("k,n_sink,n_local", [(0, 1, 1), (0, 0, 1), (3, 0, 0), (2, 4, 4)])
def test_budget_edges(k, n_sink, n_local):
    sp = W.spec("gqa_bf16", batch=4, lengths=("list", (1, 40, 200, 333)))
    w = on_gpu(W.make(sp, "cpu", seed=4))
    pipeline_check(w, range(4), DecodeStep(w, k=k, n_sink=n_sink, n_local=n_local))


def test_zero_query_selects_lowest_indices():
    sp = W.spec("gqa_bf16", batch=3, lengths=("list", (300, 517, 64)))
    w = on_gpu(W.make(sp, "cpu", seed=5))
    w.q.zero_()
    step, refs, differing = pipeline_check(w, range(3))
    assert differing == 0
    sel = step.sel.cpu().numpy()
    for b in range(3):
        n = w.n_pages(b)
        for g in range(w.spec.num_kv_heads):
            want = sorted(set(range(min(n, 1 + 16))) | {n - 1})
            assert list(sel[b, g][:len(want)]) == want


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
@pytest.mark.parametrize("base", ["longgen_bf16", "mla_bf16", "tiny_fp32"])
def test_split_count_invariance(base, splits):
    lens = {"longgen_bf16": ("uniform", 2500, 3000), "mla_bf16": ("uniform", 4000, 5000),
            "tiny_fp32": ("uniform", 500, 1000)}[base]
    sp = W.spec(base, batch=3, lengths=lens, headroom_tokens=0, pool=("factor", 1.25))
    w = on_gpu(W.make(sp, "cpu", seed=6))
    pipeline_check(w, range(3), DecodeStep(w, num_splits=splits))


def test_deterministic_and_layout_invariant():
    sp = W.spec("gqa_bf16", batch=4, lengths=("uniform", 300, 900))
    w = on_gpu(W.make(sp, "cpu", seed=7))
    a = DecodeStep(w)
    a.rebuild_centroids(); a.run(); T.sync()
    first = [t.clone() for t in (a.scores, a.sel, a.sel_count, a.out, a.lse)]
    a.run(); T.sync()
    for x, y in zip(first, (a.scores, a.sel, a.sel_count, a.out, a.lse)):
        assert torch.equal(x, y)
    # the same logical data under another page table gives the same bits
    perm = np.random.default_rng(8).permutation(w.pool_pages)
    d_perm = torch.from_numpy(perm.astype(np.int64)).cuda()
    k2 = torch.empty_like(w.k_pool); k2[d_perm] = w.k_pool
    v2 = torch.empty_like(w.v_pool); v2[d_perm] = w.v_pool
    w2 = W.Workload(spec=w.spec, device=w.device, seq_lens=w.seq_lens.copy(),
                    indptr=w.indptr.copy(), page_ids=perm[w.page_ids].astype(np.int32),
                    pool_pages=w.pool_pages, q=w.q.clone(), k_pool=k2, v_pool=v2,
                    rand_u32=w.rand_u32.copy())
    c = DecodeStep(w2)
    c.rebuild_centroids(); c.run(); T.sync()
    assert torch.equal(a.scores, c.scores)
    assert torch.equal(a.sel, c.sel) and torch.equal(a.out, c.out) and torch.equal(a.lse, c.lse)
    assert torch.equal(a.centroids[torch.from_numpy(w.page_ids.astype(np.int64)).cuda()],
                       c.centroids[torch.from_numpy(w2.page_ids.astype(np.int64)).cuda()])


@pytest.mark.parametrize("base", ["longgen_bf16", "tiny_fp32"])
def test_append_refresh_equals_rebuild(base):
    """Appending tokens and refreshing only the newest page reproduces a full
    rebuild bit for bit, across page boundaries; the step then matches the
    oracle at the new lengths."""
    extra = 40
    if base == "tiny_fp32":
        sp = W.spec(base, lengths=("fixed", 1000), headroom_tokens=extra, pool=("fixed", 128))
    else:
        sp = W.spec(base, batch=3, lengths=("list", (1000, 1007, 1023)), headroom_tokens=extra)
    w = on_gpu(W.make(sp, "cpu", seed=9))
    step = DecodeStep(w)
    step.rebuild_centroids()
    for _ in range(extra):
        w.append_token()
        step.refresh_centroids()
    T.sync()
    inc = step.centroids.clone()
    step.centroids.zero_()
    step.rebuild_centroids(); T.sync()
    used = torch.from_numpy(w.page_ids.astype(np.int64)).cuda()
    assert torch.equal(inc[used], step.centroids[used])
    pipeline_check(w, range(w.batch), step)


def test_fused_slot_write():
    """k_new / v_new land in the newest token's slot and the centroid equals a
    rebuild over the written pool."""
    sp = W.spec("longgen_bf16", batch=3, lengths=("list", (500, 511, 512)), headroom_tokens=32)
    w = on_gpu(W.make(sp, "cpu", seed=10))
    step = DecodeStep(w)
    step.rebuild_centroids()
    w.append_token()
    s = w.spec
    k_new = torch.randn((s.batch, s.num_kv_heads, s.head_dim_k), device="cuda").to(torch.bfloat16)
    v_new = torch.randn((s.batch, s.num_kv_heads, s.head_dim_v), device="cuda").to(torch.bfloat16)
    step.refresh_centroids(k_new=k_new, v_new=v_new)
    T.sync()
    for b in range(s.batch):
        t = int(w.seq_lens[b]) - 1
        pid = int(w.page_ids[w.indptr[b] + t // s.page_size])
        assert torch.equal(w.k_pool[pid, :, t % s.page_size], k_new[b])
        assert torch.equal(w.v_pool[pid, :, t % s.page_size], v_new[b])
    inc = step.centroids.clone()
    step.rebuild_centroids(); T.sync()
    used = torch.from_numpy(w.page_ids.astype(np.int64)).cuda()
    assert torch.equal(inc[used], step.centroids[used])
    pipeline_check(w, range(w.batch), step)
