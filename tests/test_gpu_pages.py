"""vx_check_pages on the GPU: zero counts for the generated page tables, and
the count of each rule for tables broken on purpose (only the check kernel
reads a broken table; it reads by index, never through a checked value)."""

import numpy as np
import pytest
import torch

from sparse_attention_decode_amd import binding as V
from sparse_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

SMALL = {
    "gqa": W.spec("gqa_bf16", batch=5, lengths=("list", (300, 40, 1, 0, 700))),
    "mla": W.spec("mla_bf16", batch=3, lengths=("list", (5000, 64, 900))),
    "tiny": W.spec("tiny_fp32"),
}


def counts_of(batch, page_size, pool, indptr, page_ids, seq_lens, total=None, maxp=None):
    indptr = np.asarray(indptr, dtype=np.int32)
    d_indptr = torch.from_numpy(indptr).cuda()
    d_ids = torch.from_numpy(np.asarray(page_ids, dtype=np.int32)).cuda()
    d_lens = torch.from_numpy(np.asarray(seq_lens, dtype=np.int32)).cuda()
    total = int(len(page_ids)) if total is None else total
    caps = np.diff(indptr)
    maxp = int(max(0, caps.max(initial=0))) if maxp is None else maxp
    maxp = min(maxp, total)
    pages = V.make_pages(batch, page_size, pool, total, maxp, d_indptr, d_ids, d_lens)
    counts = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    V.vx_check_pages(pages, counts)
    torch.cuda.synchronize()
    return counts.cpu().tolist()


@pytest.mark.parametrize("name", list(SMALL))
def test_generated_tables_are_well_formed(name):
    w = W.make(SMALL[name].replace(headroom_tokens=20), "cuda", seed=3)
    pages = V.make_pages(w.batch, w.spec.page_size, w.pool_pages, w.nnz, w.max_pages,
                         w.d_indptr, w.d_page_ids, w.d_seq_lens)
    counts = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    V.vx_check_pages(pages, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 0]


def test_full_size_table_is_well_formed():
    w = W.make(W.spec("largebatch_bf16"), "cuda", seed=0)
    pages = V.make_pages(w.batch, w.spec.page_size, w.pool_pages, w.nnz, w.max_pages,
                         w.d_indptr, w.d_page_ids, w.d_seq_lens)
    counts = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    V.vx_check_pages(pages, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 0]
    del w
    torch.cuda.empty_cache()


def test_each_rule_counted():
    # three sequences of capacity 2, 3, 1 pages of 16 tokens in a 10-page pool
    indptr = [0, 2, 5, 6]
    ids = [3, 1, 0, 9, 4, 7]
    lens = [20, 33, 16]
    assert counts_of(3, 16, 10, indptr, ids, lens) == [0, 0, 0]
    # page ids outside the pool (in use and capacity alike)
    assert counts_of(3, 16, 10, indptr, [3, -1, 0, 10, 4, 12], lens) == [0, 0, 3]
    # lengths: negative, above capacity (3 pages = 48 tokens), at capacity (fine)
    assert counts_of(3, 16, 10, indptr, ids, [-1, 49, 16]) == [0, 2, 0]
    # a capacity above max_pages
    assert counts_of(3, 16, 10, indptr, ids, lens, maxp=2) == [0, 1, 0]
    # indptr decreasing (entry 2), not starting at 0, total_pages not indptr[B]
    assert counts_of(3, 16, 10, [0, 4, 2, 6], ids, [20, 0, 16])[0] == 1
    assert counts_of(3, 16, 10, [1, 2, 5, 6], ids, lens)[0] == 1
    assert counts_of(3, 16, 10, indptr, ids, lens, total=5)[0] == 1


def test_empty_batch():
    pages = V.make_pages(0, 16, 0, 0, 0, None, None, None)
    counts = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    V.vx_check_pages(pages, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 0]
