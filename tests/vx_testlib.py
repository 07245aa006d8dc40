"""Helpers of the GPU parity tests: run the HIP step, run the oracle on the
same seeded inputs, and compare with the stated tolerances.

Tolerances (written here once, used by every parity test):
* centroids: |c_gpu - c_ref| <= 1e-5 * mean_t |K[t, g, d]| per element (the
  mean of the page's valid keys; relative to the magnitude of what is summed);
* scores: |s_gpu - s_ref| <= 1e-5 * scale * sum_h sum_d |q_hd c_d| (relative to
  the condition of the dot product; a plain |ds|/|s| is ill-posed near 0);
  bound scores likewise with max(|lo_d|, |hi_d|) in place of |c_d|;
* page bounds: exact (the minimum and maximum of KV-dtype values);
* selection: bit-exact, except that a page may differ where the oracle's
  score lies within 1e-3 relative of the k-th ranked candidate score tau:
  |s(p) - tau| <= 1e-3 * max(|tau|, 1e-3 * max |s|);
* attention: max |out_gpu - out_ref| <= 1e-4 for fp32 KV, 2e-2 for bf16 KV,
  computed on the same selected pages; lse likewise.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import vx_oracle as O
from sparse_attention_decode_amd.step import DecodeStep
from sparse_attention_decode_amd import workloads as W

ATOL = {"f32": 1e-4, "bf16": 2e-2}


def oracle_seq(w: W.Workload, step: DecodeStep, b: int, approx: bool = False) -> dict:
    s = w.spec
    seq = w.host_sequence(b)
    r = O.decode_sequence(seq, page_size=s.page_size, num_kv_heads=s.num_kv_heads, k=step.k,
                          n_sink=step.n_sink, n_local=step.n_local,
                          score_scale=step.score_scale, sm_scale=step.sm_scale, mla=s.mla,
                          head_dim_v=s.head_dim_v, approx=approx,
                          score_dim=step.score_dim or None,
                          indexer=getattr(step, "indexer", "centroid"),
                          score_bf16=getattr(step, "score_bf16", False))
    r["seq"] = seq
    return r


def gpu_centroids(w, step, b, n):
    lo = int(w.indptr[b])
    ids = torch.from_numpy(w.page_ids[lo:lo + n].astype(np.int64)).to(w.device)
    return step.centroids.index_select(0, ids).double().cpu().numpy()


def check_centroids(w, step, b, ref):
    s = w.spec
    seq = ref["seq"]
    n = ref["centroids"].shape[0]
    got = gpu_centroids(w, step, b, n)
    L = seq["seq_len"]
    bound = np.zeros_like(ref["centroids"])
    for p in range(n):
        nv = O.valid_tokens(L, s.page_size, p)
        bound[p] = np.abs(seq["k"][p, :, :nv, :]).mean(axis=1)
    err = np.abs(got - ref["centroids"])
    assert np.all(err <= 1e-5 * bound + 1e-30), f"centroid err {err.max()} (b={b})"
    return got


def check_bounds(w, step, b, ref):
    """The GPU's bounds rows of sequence b's pages in use equal the oracle's
    (values compared, so -0.0 and +0.0 are alike)."""
    n = ref["lo"].shape[0]
    lo = int(w.indptr[b])
    ids = torch.from_numpy(w.page_ids[lo:lo + n].astype(np.int64)).to(w.device)
    got = step.bounds.index_select(0, ids).double().cpu().numpy()  # [n][Hkv][Dk/4][2][4]
    n_, H, U = got.shape[:3]
    np.testing.assert_array_equal(got[:, :, :, 0, :].reshape(n_, H, 4 * U), ref["lo"],
                                  err_msg=f"lo b={b}")
    np.testing.assert_array_equal(got[:, :, :, 1, :].reshape(n_, H, 4 * U), ref["hi"],
                                  err_msg=f"hi b={b}")


def check_bound_scores(w, step, b, ref):
    s = w.spec
    n = ref["lo"].shape[0]
    lo = int(w.indptr[b])
    got = step.scores[:, lo:lo + n].double().cpu().numpy()
    q = ref["seq"]["q"]
    G = s.num_q_heads // s.num_kv_heads
    mag = np.maximum(np.abs(ref["lo"]), np.abs(ref["hi"]))  # [n][Hkv][Dk]
    bound = np.zeros((s.num_kv_heads, n))
    for g in range(s.num_kv_heads):
        qa = np.abs(q[g * G:(g + 1) * G]).sum(axis=0)
        bound[g] = step.score_scale * (mag[:, g, :] @ qa)
    err = np.abs(got - ref["scores"])
    assert np.all(err <= 1e-5 * bound + 1e-30), f"bound score err {err.max()} (b={b})"
    return got


def check_scores(w, step, b, ref):
    s = w.spec
    n = ref["centroids"].shape[0]
    lo = int(w.indptr[b])
    got = step.scores[:, lo:lo + n].double().cpu().numpy()
    d = step.score_dim or s.head_dim_k  # columns scored
    q = ref["seq"]["q"][:, :d]
    bf16 = s.mla or getattr(step, "score_bf16", False)
    cent = (O.round_to_bf16(ref["centroids"]) if bf16 else ref["centroids"])[..., :d]
    G = s.num_q_heads // s.num_kv_heads
    bound = np.zeros((s.num_kv_heads, n))
    for g in range(s.num_kv_heads):
        bound[g] = step.score_scale * (np.abs(q[g * G:(g + 1) * G]) @ np.abs(cent[:, g, :]).T).sum(0)
    err = np.abs(got - ref["scores"])
    assert np.all(err <= 1e-5 * bound + 1e-30), f"score err {err.max()} (b={b})"
    return got


def near_tie_ok(sel_gpu, sel_ref, scores_ref, n, k, n_sink, n_local) -> tuple[bool, int]:
    """Selections must match, except pages whose oracle score is within 1e-3
    relative of tau (the k-th ranked candidate score). Returns (ok, #diffs)."""
    a = set(int(x) for x in sel_gpu if x >= 0)
    r = set(int(x) for x in sel_ref if x >= 0)
    if a == r:
        return True, 0
    if len(a) != len(r):
        return False, len(a ^ r)
    forced = set(O.forced_pages(n, n_sink, n_local))
    cand = [p for p in range(n) if p not in forced]
    ranked = sorted(cand, key=lambda p: (-scores_ref[p], p))
    tau = scores_ref[ranked[min(k, len(ranked)) - 1]]
    smax = max(abs(scores_ref[p]) for p in cand)
    band = 1e-3 * max(abs(tau), 1e-3 * smax)
    diff = a ^ r
    ok = all(p in cand and abs(scores_ref[p] - tau) <= band for p in diff)
    return ok, len(diff)


def check_selection(w, step, b, ref):
    s = w.spec
    n = ref["centroids"].shape[0]
    sel = step.sel[b].cpu().numpy()
    cnt = step.sel_count[b].cpu().numpy()
    same = []
    for g in range(s.num_kv_heads):
        got = sel[g]
        assert cnt[g] == int((ref["sel"][g] >= 0).sum()), (b, g, cnt[g])
        ids = got[:cnt[g]]
        assert np.all(np.diff(ids) > 0) and np.all(got[cnt[g]:] == -1), (b, g, got)
        ok, nd = near_tie_ok(got, ref["sel"][g], ref["scores"][g], n, step.k, step.n_sink,
                             step.n_local)
        assert ok, (b, g, got, ref["sel"][g])
        same.append(nd == 0)
    return same


def check_attention(w, out_gpu, lse_gpu, out_ref, lse_ref, heads=None, tag=""):
    atol = ATOL[w.spec.kv_dtype]
    hs = range(out_ref.shape[0]) if heads is None else heads
    for h in hs:
        e = np.abs(out_gpu[h] - out_ref[h]).max()
        assert e <= atol, f"out err {e} > {atol} head {h} {tag}"
        if lse_gpu is not None:
            if np.isinf(lse_ref[h]):
                assert np.isinf(lse_gpu[h]) and lse_gpu[h] < 0
            else:
                el = abs(lse_gpu[h] - lse_ref[h])
                assert el <= atol, f"lse err {el} head {h} {tag}"


def sel_tensor_from_oracle(w, step, refs: dict) -> tuple[torch.Tensor, torch.Tensor]:
    """Device sel / sel_count holding the oracle's selections (to run the GPU
    attention on exactly the oracle's pages)."""
    s = w.spec
    sel = torch.full((s.batch, s.num_kv_heads, step.k_out), -1, dtype=torch.int32)
    cnt = torch.zeros((s.batch, s.num_kv_heads), dtype=torch.int32)
    for b, r in refs.items():
        for g in range(s.num_kv_heads):
            ids = [int(x) for x in r["sel"][g] if x >= 0]
            sel[b, g, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
            cnt[b, g] = len(ids)
    return sel.to(w.device), cnt.to(w.device)


def oracle_attention_on(w, step, ref):
    """The oracle's attention for one sequence, on its own selection."""
    return ref["out"], ref["lse"]


def check_attention_on_gpu_selection(w, step, b, ref, out_b, lse_b, g=None, tag=""):
    """Where a near tie made the GPU's selection differ from the oracle's,
    the GPU's attention is still checked: against the oracle's attention on
    the GPU's own selection (KV head g, or every head when g is None)."""
    s = w.spec
    seq = ref["seq"]
    sel = step.sel[b].cpu().numpy().astype(np.int64)  # [Hkv][K_out], -1 padded
    vv = seq["k"][..., :s.head_dim_v] if s.mla else seq["v"]
    out_ref, lse_ref = O.attention(seq["q"], seq["k"], vv, seq["seq_len"], s.page_size, sel,
                                   step.sm_scale, s.num_kv_heads)
    G = s.num_q_heads // s.num_kv_heads
    heads = None if g is None else range(g * G, (g + 1) * G)
    check_attention(w, out_b, lse_b, out_ref, lse_ref, heads=heads,
                    tag=f"{tag} (on the GPU's selection)")


def sync():
    torch.cuda.synchronize()
