"""Seeded synthetic inputs for one block top-k sparse-attention decode step.

This module draws random numbers and builds paged-KV metadata. It holds none
of the method's arithmetic (no centroid, score, selection or attention math):
both the HIP path and the CPU oracle consume what it produces.

Page layout (the paged KV cache of the Vortex paper note, papers.chlience.com,
section "System design > 2. vTensor": a tensor plus batch size, a pointer array
and a page-index structure):

* ``indptr[B+1]``  pointer array; sequence ``b`` owns page-table entries
  ``indptr[b] .. indptr[b+1]-1`` (its capacity, which may exceed the pages in
  use so that appended tokens have a slot),
* ``page_ids[nnz]`` physical page of each logical page,
* ``seq_lens[B]``   valid tokens of each sequence,
* ``k_pool[pool][Hkv][P][Dk]``, ``v_pool[pool][Hkv][P][Dv]`` (MLA: one latent
  stream, ``Hkv == 1``, no separate V pool; V is the first ``Dv`` columns of K).

The five named workloads and their input recipes:

``tiny_fp32``        B=1, Hq=2, Hkv=1, D=64, P=16, L=1024 in a 128-page pool
                     under a random permutation; fp32; q, K, V iid N(0,1);
                     top-8 plus the last page.
``gqa_bf16``         B=32, Hq=16, Hkv=8, D=128, P=16, L ~ U[2048, 4096]; pool
                     1.25x the pages used, scattered at random; bf16; q, K, V
                     N(0,1); 5% of token positions per sequence get +3 along a
                     unit direction drawn once per KV head; top-16 + sink + last.
``longgen_bf16``     B=64, Hq=32, Hkv=8, D=128, P=16, L ~ U[8192, 32768]; bf16;
                     per (sequence, KV head) the page key mean follows a random
                     walk mu_0 = 0, mu_{p+1} = mu_p + 0.1 xi_p, xi ~ N(0, I);
                     key = mu_page + N(0, I); top-128 + sink + last 2 pages;
                     page tables carry headroom for appended tokens.
``mla_bf16``         B=32, Hq=32 over one 576-wide latent stream (512 latent +
                     64 rope), Dv=512, P=64, L ~ U[16384, 65536]; latent columns
                     0.5 N(0,1), rope columns N(0,1), for both q and K;
                     top-32 + sink + last.
``largebatch_bf16``  B=256, Hq=64, Hkv=8, D=128, P=64, L lognormal with median
                     16384 and sigma ln 2, clipped to [4096, 65536]; bf16;
                     q, K, V N(0,1); top-64, no forced pages.

Every draw is seeded (seed 0 by default). Metadata and the per-segment random
words of the stochastic top-k come from a NumPy PCG64 stream, tensors from a
``torch.Generator`` on the device they are built on.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Spec", "Workload", "SPECS", "make", "spec"]


@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    page_size: int
    # ("fixed", L) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    # | ("list", (L_0, ..., L_{B-1}))
    lengths: tuple
    # ("fixed", pages) | ("factor", f)
    pool: tuple
    kv_dtype: str  # "f32" | "bf16"
    q_dtype: str
    topk: int
    n_sink: int
    n_local: int
    key_model: str  # "iid" | "boost" | "walk" | "mla"
    mla: bool = False
    headroom_tokens: int = 0  # extra page-table capacity per sequence
    score_scale: Optional[float] = None  # default 1/sqrt(Dk)
    sm_scale: Optional[float] = None  # default 1/sqrt(Dk)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def k_out(self) -> int:
        return self.topk + self.n_sink + self.n_local

    def scales(self) -> tuple[float, float]:
        d = 1.0 / math.sqrt(self.head_dim_k)
        return (self.score_scale if self.score_scale is not None else d,
                self.sm_scale if self.sm_scale is not None else d)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


SPECS: dict[str, Spec] = {
    "tiny_fp32": Spec(
        name="tiny_fp32", batch=1, num_q_heads=2, num_kv_heads=1,
        head_dim_k=64, head_dim_v=64, page_size=16, lengths=("fixed", 1024),
        pool=("fixed", 128), kv_dtype="f32", q_dtype="f32", topk=8,
        n_sink=0, n_local=1, key_model="iid"),
    "gqa_bf16": Spec(
        name="gqa_bf16", batch=32, num_q_heads=16, num_kv_heads=8,
        head_dim_k=128, head_dim_v=128, page_size=16,
        lengths=("uniform", 2048, 4096), pool=("factor", 1.25),
        kv_dtype="bf16", q_dtype="bf16", topk=16, n_sink=1, n_local=1,
        key_model="boost"),
    "longgen_bf16": Spec(
        name="longgen_bf16", batch=64, num_q_heads=32, num_kv_heads=8,
        head_dim_k=128, head_dim_v=128, page_size=16,
        lengths=("uniform", 8192, 32768), pool=("factor", 1.25),
        kv_dtype="bf16", q_dtype="bf16", topk=128, n_sink=1, n_local=2,
        key_model="walk", headroom_tokens=64),
    "mla_bf16": Spec(
        name="mla_bf16", batch=32, num_q_heads=32, num_kv_heads=1,
        head_dim_k=576, head_dim_v=512, page_size=64,
        lengths=("uniform", 16384, 65536), pool=("factor", 1.25),
        kv_dtype="bf16", q_dtype="bf16", topk=32, n_sink=1, n_local=1,
        key_model="mla", mla=True),
    "largebatch_bf16": Spec(
        name="largebatch_bf16", batch=256, num_q_heads=64, num_kv_heads=8,
        head_dim_k=128, head_dim_v=128, page_size=64,
        lengths=("lognormal", 16384, math.log(2.0), 4096, 65536),
        pool=("factor", 1.25), kv_dtype="bf16", q_dtype="bf16", topk=64,
        n_sink=0, n_local=0, key_model="iid"),
}

MLA_LATENT = 512  # columns 0..511 latent, 512..575 rope
_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def spec(name: str, **overrides) -> Spec:
    s = SPECS[name]
    return s.replace(**overrides) if overrides else s


@dataclass
class Workload:
    spec: Spec
    device: torch.device
    seq_lens: np.ndarray  # int32 [B], host copy
    indptr: np.ndarray  # int32 [B+1], host copy
    page_ids: np.ndarray  # int32 [nnz], host copy
    pool_pages: int
    q: torch.Tensor  # [B][Hq][Dk]
    k_pool: torch.Tensor  # [pool][Hkv][P][Dk]
    v_pool: Optional[torch.Tensor]  # [pool][Hkv][P][Dv] or None (MLA)
    rand_u32: np.ndarray  # uint32 [B][Hkv]: draws for the stochastic top-k
    d_seq_lens: torch.Tensor = field(repr=False, default=None)
    d_indptr: torch.Tensor = field(repr=False, default=None)
    d_page_ids: torch.Tensor = field(repr=False, default=None)
    d_rand_u32: torch.Tensor = field(repr=False, default=None)

    def __post_init__(self):
        self._upload_meta()

    def _upload_meta(self):
        dev = self.device
        self.d_seq_lens = torch.from_numpy(self.seq_lens.astype(np.int32)).to(dev)
        self.d_indptr = torch.from_numpy(self.indptr.astype(np.int32)).to(dev)
        self.d_page_ids = torch.from_numpy(self.page_ids.astype(np.int32)).to(dev)
        self.d_rand_u32 = torch.from_numpy(
            self.rand_u32.astype(np.uint32).view(np.int32)).to(dev)

    # ---- host-side sizes -------------------------------------------------
    @property
    def batch(self) -> int:
        return self.spec.batch

    @property
    def nnz(self) -> int:
        return int(self.indptr[-1])

    @property
    def max_pages(self) -> int:
        return int(np.max(np.diff(self.indptr))) if self.batch else 0

    def n_pages(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.spec.page_size)

    # ---- growth (appending one token per sequence) -----------------------
    def append_token(self) -> None:
        """Grow every sequence by one token. The token's K/V already sit in
        the pool slot (drawn at construction for the page-table headroom)."""
        P = self.spec.page_size
        cap = np.diff(self.indptr) * P
        if np.any(self.seq_lens + 1 > cap):
            raise ValueError("page-table headroom exhausted")
        self.seq_lens = (self.seq_lens + 1).astype(np.int32)
        self.d_seq_lens.copy_(torch.from_numpy(self.seq_lens))

    # ---- copies for the oracle ------------------------------------------
    def host_sequence(self, b: int) -> dict:
        """float64 host copies of one sequence, pages in logical order:
        q [Hq][Dk], k [cap][Hkv][P][Dk], v [cap][Hkv][P][Dv] (MLA: None)."""
        lo, hi = int(self.indptr[b]), int(self.indptr[b + 1])
        ids = torch.from_numpy(self.page_ids[lo:hi].astype(np.int64)).to(self.device)
        k = self.k_pool.index_select(0, ids).float().cpu().double().numpy()
        v = None
        if self.v_pool is not None:
            v = self.v_pool.index_select(0, ids).float().cpu().double().numpy()
        return {
            "q": self.q[b].float().cpu().double().numpy(),
            "k": k,
            "v": v,
            "seq_len": int(self.seq_lens[b]),
            "rand_u32": self.rand_u32[b].astype(np.uint32),
        }

    def replicate(self) -> "Workload":
        """A copy in fresh device memory (same values, different addresses)."""
        return Workload(
            spec=self.spec, device=self.device, seq_lens=self.seq_lens.copy(),
            indptr=self.indptr.copy(), page_ids=self.page_ids.copy(),
            pool_pages=self.pool_pages, q=self.q.clone(),
            k_pool=self.k_pool.clone(),
            v_pool=None if self.v_pool is None else self.v_pool.clone(),
            rand_u32=self.rand_u32.copy())


def _lengths(s: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = s.lengths[0]
    if kind == "list":
        lens = np.asarray(s.lengths[1], dtype=np.int64)
        if lens.shape != (s.batch,):
            raise ValueError("length list does not match the batch")
        return lens
    if kind == "fixed":
        return np.full(s.batch, s.lengths[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(s.lengths[1], s.lengths[2] + 1, size=s.batch)
    if kind == "lognormal":
        median, sigma, lo, hi = s.lengths[1:]
        x = np.exp(math.log(median) + sigma * rng.standard_normal(s.batch))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(kind)


def _randn(shape, gen, device, scale=None, chunk_rows=4096) -> torch.Tensor:
    """fp32 normal draws, built in row chunks to bound peak memory."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        blk = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen,
                          device=device, dtype=torch.float32)
        if scale is not None:
            blk.mul_(scale)
        out[r0:r1] = blk
    return out


def _randn_cast(shape, gen, device, dtype, scale=None, chunk_rows=2048):
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        blk = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen,
                          device=device, dtype=torch.float32)
        if scale is not None:
            blk.mul_(scale)
        out[r0:r1] = blk.to(dtype)
    return out


def make(s: Spec, device="cpu", seed: int = 0) -> Workload:
    """Build the seeded workload ``s`` with its tensors on ``device``."""
    device = torch.device(device)
    rng = np.random.default_rng(seed)
    B, Hq, Hkv = s.batch, s.num_q_heads, s.num_kv_heads
    P, Dk, Dv = s.page_size, s.head_dim_k, s.head_dim_v
    if s.mla and Hkv != 1:
        raise ValueError("the MLA geometry has one latent KV stream")

    lens = _lengths(s, rng)
    cap = -(-(lens + s.headroom_tokens) // P)
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(cap)
    nnz = int(indptr[-1])
    if s.pool[0] == "fixed":
        pool = int(s.pool[1])
    else:
        pool = max(nnz, int(math.ceil(s.pool[1] * nnz)))
    if pool < nnz:
        raise ValueError("pool smaller than the page tables")
    page_ids = rng.permutation(pool)[:nnz]
    rand_u32 = rng.integers(0, 2**32, size=(B, Hkv), dtype=np.uint64).astype(np.uint32)

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    kv_dt = _TORCH_DTYPES[s.kv_dtype]
    q_dt = _TORCH_DTYPES[s.q_dtype]

    col_scale = None
    if s.key_model == "mla":
        col_scale = torch.ones(Dk, dtype=torch.float32, device=device)
        col_scale[:MLA_LATENT] = 0.5

    k_pool = _randn_cast((pool, Hkv, P, Dk), gen, device, kv_dt, col_scale)
    v_pool = None if s.mla else _randn_cast((pool, Hkv, P, Dv), gen, device, kv_dt)
    q = _randn((B, Hq, Dk), gen, device, col_scale).to(q_dt)

    d_ids = torch.from_numpy(page_ids.astype(np.int64)).to(device)
    if s.key_model == "boost":
        # one unit direction per KV head, shared by every sequence
        u = torch.randn((Hkv, Dk), generator=gen, device=device, dtype=torch.float32)
        u = u / u.norm(dim=1, keepdim=True)
        pages, slots = [], []
        for b in range(B):
            L = int(lens[b])
            m = int(np.rint(0.05 * L))
            pos = rng.choice(L, size=m, replace=False)
            pages.append(page_ids[indptr[b] + pos // P])
            slots.append(pos % P)
        pg = torch.from_numpy(np.concatenate(pages).astype(np.int64)).to(device)
        sl = torch.from_numpy(np.concatenate(slots).astype(np.int64)).to(device)
        rows = k_pool[pg, :, sl, :].float() + 3.0 * u  # [n][Hkv][Dk]
        k_pool[pg, :, sl, :] = rows.to(kv_dt)
    elif s.key_model == "walk":
        # random-walk page means per (sequence, KV head), mu_0 = 0
        steps = 0.1 * _randn((nnz, Hkv, Dk), gen, device).double()
        starts = torch.from_numpy(indptr[:-1].astype(np.int64)).to(device)
        steps[starts] = 0.0
        csum = torch.cumsum(steps, dim=0)
        seg = torch.from_numpy(np.repeat(np.arange(B), cap).astype(np.int64)).to(device)
        mu = (csum - csum[starts][seg]).float()  # [nnz][Hkv][Dk]
        for j0 in range(0, nnz, 8192):
            j1 = min(nnz, j0 + 8192)
            ids = d_ids[j0:j1]
            blk = k_pool[ids].float() + mu[j0:j1, :, None, :]
            k_pool[ids] = blk.to(kv_dt)
        del steps, csum, mu

    return Workload(
        spec=s, device=device, seq_lens=lens.astype(np.int32),
        indptr=indptr.astype(np.int32), page_ids=page_ids.astype(np.int32),
        pool_pages=pool, q=q, k_pool=k_pool, v_pool=v_pool,
        rand_u32=rand_u32)
