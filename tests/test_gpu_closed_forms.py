"""Closed forms of the whole step at full size, in the launch configuration
the benchmark times (vx_decode_step: the one-kernel GQA step, the MLA
scorer + split attention + merge, and a forced split GQA step), for every
workload.

With q = 0 every page scores 0 and every logit is 0, so, from the method's
definition (Vortex paper note, "System design > 1. vFlow": top-k blocks by
score, then exact softmax attention over them):
* the selection is the forced pages plus the first min(k, #candidates)
  other pages by index (the tie-break), or, in approximate mode, the
  candidates whose rank falls in the cyclic window of length kk starting at
  rand mod #candidates (every candidate falls into one bucket);
* lse = ln T for every query head, T the valid tokens of its KV head's
  selection, so one token dropped or counted twice moves lse by about 1/T
  (5e-4 at T = 2176), far above the 1e-5 checked here;
* out = the mean of the selected tokens' value rows.
"""

import math

import numpy as np
import pytest
import torch

from sparse_attention_decode_amd import binding as V
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep

pytestmark = pytest.mark.gpu


def expected_selection(n, k, n_sink, n_local, approx, rnd, k_out):
    forced = sorted(set(range(min(n, n_sink))) | set(range(max(0, n - n_local), n)))
    cand = [p for p in range(n) if p not in forced]
    kk = min(k, len(cand))
    if approx and 0 < kk < len(cand):
        off = int(rnd) % len(cand)
        chosen = [cand[(off + i) % len(cand)] for i in range(kk)]
    else:
        chosen = cand[:kk]
    ids = sorted(forced + chosen)
    return ids + [-1] * (k_out - len(ids))


@pytest.mark.parametrize("name,splits,mode", [
    ("tiny_fp32", 0, V.VX_TOPK_EXACT),
    ("gqa_bf16", 0, V.VX_TOPK_EXACT),
    ("gqa_bf16", 3, V.VX_TOPK_EXACT),
    ("longgen_bf16", 0, V.VX_TOPK_EXACT),
    ("mla_bf16", 0, V.VX_TOPK_EXACT),
    ("largebatch_bf16", 0, V.VX_TOPK_EXACT),
    ("largebatch_bf16", 0, V.VX_TOPK_APPROX),
])
def test_zero_query_closed_form(name, splits, mode):
    s = W.spec(name)
    w = W.make(s, "cuda", seed=0)
    w.q.zero_()
    step = DecodeStep(w, num_splits=splits, mode=mode)
    step.rebuild()
    step.run()
    torch.cuda.synchronize()
    if splits:
        assert step.plan()["num_splits"] == splits
    P, H = s.page_size, s.num_kv_heads
    G = s.num_q_heads // H
    sel = step.sel.cpu().numpy()
    cnt = step.sel_count.cpu().numpy()
    lse = step.lse.cpu().double().numpy()
    # every segment: the selection, its count and every head's lse
    T = np.zeros((s.batch, H))
    for b in range(s.batch):
        L, n = int(w.seq_lens[b]), w.n_pages(b)
        for g in range(H):
            want = expected_selection(n, step.k, step.n_sink, step.n_local,
                                      mode == V.VX_TOPK_APPROX, w.rand_u32[b, g], step.k_out)
            np.testing.assert_array_equal(sel[b, g], want, err_msg=f"{name} b={b} g={g}")
            ids = np.array([p for p in want if p >= 0], dtype=np.int64)
            assert cnt[b, g] == len(ids)
            T[b, g] = np.clip(L - ids * P, 0, P).sum()
    want_lse = np.log(np.repeat(T, G, axis=1))
    err = np.abs(lse - want_lse)
    assert err.max() <= 1e-5, f"{name}: lse err {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"
    # sampled sequences: out is the mean of the selected value rows (fp64 torch)
    out = step.out.double()
    Dv = s.head_dim_v
    for b in sorted({0, s.batch // 2, s.batch - 1}):
        L = int(w.seq_lens[b])
        lo = int(w.indptr[b])
        for g in range(H):
            rows = []
            for p in sel[b, g, :cnt[b, g]]:
                phys = int(w.page_ids[lo + int(p)])
                nv = min(P, L - int(p) * P)
                src = w.k_pool[phys, 0, :nv, :Dv] if s.mla else w.v_pool[phys, g, :nv, :]
                rows.append(src.double())
            mean = torch.cat(rows).mean(0)
            got = out[b, g * G:(g + 1) * G]
            e = (got - mean).abs().max().item()
            assert e <= 2e-5, f"{name} b={b} g={g}: out err {e}"
    del w, step
    torch.cuda.empty_cache()
