"""Seeded random configurations (batch, lengths including idle slots and
one-token sequences, page size, head geometry, dtype, budget, forced pages,
indexer, top-k mode, appends) through the whole step against the oracle."""

import numpy as np
import pytest

import vx_testlib as T
from sparse_attention_decode_amd import binding as V
from sparse_attention_decode_amd import workloads as W
from sparse_attention_decode_amd.step import DecodeStep
from test_gpu_edges import on_gpu

pytestmark = pytest.mark.gpu


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 7))
    P = int(rng.choice([16, 64]))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    dk = int(rng.choice([64, 128]))
    dt = str(rng.choice(["bf16", "f32"]))
    lens = [int(x) for x in rng.integers(1, 3000, size=batch)]
    if batch > 2:
        lens[int(rng.integers(batch))] = 0  # an idle slot
    if batch > 1:
        lens[int(rng.integers(batch))] = 1
    k = int(rng.integers(0, 40))
    n_sink, n_local = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    indexer = "bounds" if dt == "bf16" and rng.random() < 0.4 else "centroid"
    mode = V.VX_TOPK_EXACT  # the oracle's approximate selection needs bit-identical scores
    splits = int(rng.choice([0, 0, 1, 3]))
    sp = W.spec("gqa_bf16", batch=batch, num_q_heads=hkv * G, num_kv_heads=hkv, head_dim_k=dk,
                head_dim_v=dk, page_size=P, kv_dtype=dt, q_dtype=dt, lengths=("list", tuple(lens)),
                headroom_tokens=int(rng.integers(0, 40)), pool=("factor", 1.5))
    return sp, dict(k=k, n_sink=n_sink, n_local=n_local, indexer=indexer, mode=mode,
                    num_splits=splits), int(rng.integers(0, 4))


@pytest.mark.parametrize("seed", range(40))
def test_random_configuration(seed):
    sp, kw, appends = random_case(seed)
    w = on_gpu(W.make(sp, "cpu", seed=seed))
    step = DecodeStep(w, **kw)
    step.rebuild()
    step.run()
    for _ in range(min(appends, sp.headroom_tokens)):
        w.append_token()
        step.run()
    T.sync()
    out = step.out.cpu().double().numpy()
    lse = step.lse.cpu().double().numpy()
    G = sp.num_q_heads // sp.num_kv_heads
    differing = 0
    for b in range(sp.batch):
        if int(w.seq_lens[b]) == 0:
            assert (step.out[b] == 0).all() and (step.sel_count[b] == 0).all()
            continue
        r = T.oracle_seq(w, step, b)
        if kw["indexer"] == "bounds":
            T.check_bounds(w, step, b, r)
            T.check_bound_scores(w, step, b, r)
        else:
            T.check_centroids(w, step, b, r)
            T.check_scores(w, step, b, r)
        for g, ok in enumerate(T.check_selection(w, step, b, r)):
            if ok:
                T.check_attention(w, out[b], lse[b], r["out"], r["lse"],
                                  heads=range(g * G, (g + 1) * G), tag=f"seed={seed} b={b} g={g}")
            else:
                differing += 1
                T.check_attention_on_gpu_selection(w, step, b, r, out[b], lse[b], g,
                                                   tag=f"seed={seed} b={b} g={g}")
    assert differing <= 1


@pytest.mark.parametrize("seed", range(10))
def test_random_mla_configuration(seed):
    rng = np.random.default_rng(2000 + seed)
    batch = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 9000, size=batch)]
    if batch > 2:
        lens[int(rng.integers(batch))] = 0
    hq = int(rng.choice([16, 32]))
    sp = W.spec("mla_bf16", batch=batch, num_q_heads=hq, lengths=("list", tuple(lens)),
                headroom_tokens=int(rng.integers(0, 70)), pool=("factor", 1.5))
    kw = dict(k=int(rng.integers(0, 40)), n_sink=int(rng.integers(0, 3)),
              n_local=int(rng.integers(0, 3)), num_splits=int(rng.choice([0, 0, 1, 5])),
              score_dim=int(rng.choice([0, 512])))
    w = on_gpu(W.make(sp, "cpu", seed=seed))
    step = DecodeStep(w, **kw)
    step.rebuild()
    step.run()
    for _ in range(min(int(rng.integers(0, 3)), sp.headroom_tokens)):
        w.append_token()
        step.run()
    T.sync()
    out = step.out.cpu().double().numpy()
    lse = step.lse.cpu().double().numpy()
    differing = 0
    for b in range(batch):
        if int(w.seq_lens[b]) == 0:
            assert (step.out[b] == 0).all() and (step.sel_count[b] == 0).all()
            continue
        r = T.oracle_seq(w, step, b)
        T.check_centroids(w, step, b, r)
        T.check_scores(w, step, b, r)
        if T.check_selection(w, step, b, r)[0]:
            T.check_attention(w, out[b], lse[b], r["out"], r["lse"], tag=f"seed={seed} b={b}")
        else:
            differing += 1
            T.check_attention_on_gpu_selection(w, step, b, r, out[b], lse[b],
                                               tag=f"seed={seed} b={b}")
    assert differing <= 1
