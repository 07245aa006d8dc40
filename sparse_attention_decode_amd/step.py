"""One block top-k sparse-attention decode step on the GPU.

Owns the device buffers of a workload (centroid cache, scores, selection,
outputs, workspace) and issues the library's calls in the step's order:
cache stage (refresh of the newest token's page), scoring, selection,
attention. Python only marshals arguments; every stage is a gfx950 kernel.

indexer="bounds" swaps the centroid cache stage and scorer for the
Quest-style page bounds (vx_bounds_update / vx_bound_scores, GQA only);
selection and attention are unchanged. score_bf16=True (GQA, bf16 KV)
scores the pages on the centroids' bf16 copy (MLA always does).
"""

from __future__ import annotations

from typing import Optional

import torch

from . import binding as V
from .workloads import Workload

__all__ = ["DecodeStep"]


class DecodeStep:
    def __init__(self, w: Workload, mode: int = V.VX_TOPK_EXACT, num_splits: int = 0,
                 k: Optional[int] = None, n_sink: Optional[int] = None,
                 n_local: Optional[int] = None, with_lse: bool = True, fused: bool = True,
                 score_dim: int = 0, indexer: str = "centroid", score_bf16: bool = False):
        if indexer not in ("centroid", "bounds"):
            raise ValueError(f"indexer {indexer!r}")
        s = w.spec
        dev = w.device
        self.w = w
        self.mode = mode
        self.fused = fused
        self.indexer = indexer
        self.num_splits = num_splits
        self.k = s.topk if k is None else k
        self.n_sink = s.n_sink if n_sink is None else n_sink
        self.n_local = s.n_local if n_local is None else n_local
        self.k_out = max(1, self.k + self.n_sink + self.n_local)
        self.score_scale, self.sm_scale = s.scales()
        self.pages = V.make_pages(s.batch, s.page_size, w.pool_pages, w.nnz, w.max_pages,
                                  w.d_indptr, w.d_page_ids, w.d_seq_lens)
        self.score_dim = score_dim
        self.score_bf16 = bool(score_bf16) and not s.mla
        self.geom = V.make_geom(s.num_q_heads, s.num_kv_heads, s.head_dim_k, s.head_dim_v,
                                s.mla, w.q.dtype, w.k_pool.dtype, score_dim, self.score_bf16)
        H = s.num_kv_heads
        self.centroids = torch.zeros((w.pool_pages, H, s.head_dim_k), dtype=torch.float32,
                                     device=dev)
        self.cent_bf16 = (torch.zeros((w.pool_pages, H, s.head_dim_k), dtype=torch.bfloat16,
                                      device=dev) if s.mla or self.score_bf16 else None)
        # [pool][Hkv][Dk/4][2][4]: per 4 dims, their 4 key minima then 4 maxima
        self.bounds = (torch.zeros((w.pool_pages, H, s.head_dim_k // 4, 2, 4),
                                   dtype=w.k_pool.dtype, device=dev)
                       if indexer == "bounds" else None)
        self.scores = torch.zeros((H, max(1, w.nnz)), dtype=torch.float32, device=dev)
        self.sel = torch.full((s.batch, H, self.k_out), -1, dtype=torch.int32, device=dev)
        self.sel_count = torch.zeros((s.batch, H), dtype=torch.int32, device=dev)
        self.out = torch.zeros((s.batch, s.num_q_heads, s.head_dim_v), dtype=torch.float32,
                               device=dev)
        self.lse = (torch.zeros((s.batch, s.num_q_heads), dtype=torch.float32, device=dev)
                    if with_lse else None)
        # -1: refresh the page holding each sequence's newest token
        self.newest = torch.full((s.batch,), -1, dtype=torch.int32, device=dev)
        # the whole step's workspace covers the attention's (and, for ordered
        # plans, the sequence order)
        nbytes = max(
            V.vx_sparse_decode(self.pages, self.geom, None, None, None, None, self.k_out,
                               None, self.sm_scale, None, None, num_splits),
            V.vx_decode_step(self.pages, self.geom, None, None, None, None, None, True,
                             self.score_scale, self.sm_scale, self.k, self.n_sink, self.n_local,
                             mode, None, None, None, self.k_out, None, None, None, num_splits))
        self.workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev)
        self.workspace_bytes = nbytes
        self.k_new = self.v_new = None  # appended token's K/V (append_kv draws them)

    # -- stages ---------------------------------------------------------
    def rebuild_centroids(self, stream=None) -> None:
        w = self.w
        V.vx_centroid_update(self.pages, self.geom, w.k_pool, None, None, None, None,
                             self.centroids, self.cent_bf16, stream)

    def refresh_centroids(self, first_token=None, k_new=None, v_new=None, stream=None) -> None:
        w = self.w
        ft = self.newest if first_token is None else first_token
        V.vx_centroid_update(self.pages, self.geom, w.k_pool, w.v_pool if v_new is not None else None,
                             ft, k_new, v_new, self.centroids, self.cent_bf16, stream)

    def rebuild_bounds(self, stream=None) -> None:
        V.vx_bounds_update(self.pages, self.geom, self.w.k_pool, None, self.bounds, stream)

    def refresh_bounds(self, first_token=None, stream=None) -> None:
        ft = self.newest if first_token is None else first_token
        V.vx_bounds_update(self.pages, self.geom, self.w.k_pool, ft, self.bounds, stream)

    def bound_score(self, refresh: bool = False, stream=None) -> None:
        V.vx_bound_scores(self.pages, self.geom, self.w.q, self.w.k_pool, self.bounds, refresh,
                          self.score_scale, self.scores, stream)

    def rebuild(self, stream=None) -> None:
        """Rebuild the indexer's cache from the whole pool."""
        if self.indexer == "bounds":
            self.rebuild_bounds(stream)
        else:
            self.rebuild_centroids(stream)

    def score(self, stream=None) -> None:
        cent = self.cent_bf16 if self.w.spec.mla or self.score_bf16 else self.centroids
        V.vx_page_scores(self.pages, self.geom, self.w.q, cent, self.score_scale, self.scores,
                         stream)

    def select(self, scores=None, stream=None) -> None:
        V.vx_topk_pages(self.pages, self.w.spec.num_kv_heads,
                        self.scores if scores is None else scores, self.k, self.n_sink,
                        self.n_local, self.mode, self.w.d_rand_u32, self.sel, self.k_out,
                        self.sel_count, stream)

    def index(self, refresh: bool = True, stream=None) -> None:
        """Fused indexer: newest-page refresh (optional), scores, selection."""
        w = self.w
        V.vx_index_pages(self.pages, self.geom, w.q, w.k_pool, self.centroids, self.cent_bf16,
                         refresh, self.score_scale, self.scores, self.k, self.n_sink,
                         self.n_local, self.mode, w.d_rand_u32, self.sel, self.k_out,
                         self.sel_count, stream)

    def attend(self, sel=None, sel_count=None, stream=None) -> None:
        w = self.w
        V.vx_sparse_decode(self.pages, self.geom, w.q, w.k_pool, w.v_pool,
                           self.sel if sel is None else sel, self.k_out,
                           self.sel_count if sel_count is None else sel_count, self.sm_scale,
                           self.out, self.lse, self.num_splits, self.workspace,
                           self.workspace_bytes, stream)

    def step(self, refresh: bool = True, stream=None) -> None:
        """vx_decode_step: the indexer and the attention in one call."""
        w = self.w
        V.vx_decode_step(self.pages, self.geom, w.q, w.k_pool, w.v_pool, self.centroids,
                         self.cent_bf16, refresh, self.score_scale, self.sm_scale, self.k,
                         self.n_sink, self.n_local, self.mode, w.d_rand_u32, self.scores,
                         self.sel, self.k_out, self.sel_count, self.out, self.lse,
                         self.num_splits, self.workspace, self.workspace_bytes, stream)

    def bound_step(self, refresh: bool = True, stream=None) -> None:
        """vx_bound_decode_step: the bounds indexer and the attention in one call."""
        w = self.w
        V.vx_bound_decode_step(self.pages, self.geom, w.q, w.k_pool, w.v_pool, self.bounds,
                               refresh, self.score_scale, self.sm_scale, self.k, self.n_sink,
                               self.n_local, self.mode, w.d_rand_u32, self.scores, self.sel,
                               self.k_out, self.sel_count, self.out, self.lse, self.num_splits,
                               self.workspace, self.workspace_bytes, stream)

    def _draw_new(self) -> None:
        """The appended token's K/V rows (seeded, drawn once)."""
        w = self.w
        if self.k_new is None:
            s = w.spec
            g = torch.Generator(device=w.device)
            g.manual_seed(12345)
            shape = (s.batch, s.num_kv_heads)
            self.k_new = torch.randn(shape + (s.head_dim_k,), generator=g, device=w.device).to(
                w.k_pool.dtype)
            if not s.mla:
                self.v_new = torch.randn(shape + (s.head_dim_v,), generator=g,
                                         device=w.device).to(w.k_pool.dtype)

    def append_kv(self, stream=None) -> None:
        """Cache stage of an appending decode step: write each sequence's new
        token's K/V (self.k_new / self.v_new) into the slot of its newest
        token and recompute that page's centroid (vx_centroid_update with
        first_token = -1, k_new and v_new)."""
        w = self.w
        self._draw_new()
        V.vx_centroid_update(self.pages, self.geom, w.k_pool,
                             None if w.spec.mla else w.v_pool, self.newest, self.k_new,
                             self.v_new, self.centroids, self.cent_bf16, stream)

    def append_step(self, stream=None) -> None:
        """vx_append_decode_step: the new token's K/V rows and its page's
        centroid, then the indexer and the attention, in one call (one kernel
        when the step is)."""
        w = self.w
        self._draw_new()
        V.vx_append_decode_step(self.pages, self.geom, w.q, w.k_pool,
                                None if w.spec.mla else w.v_pool, self.k_new, self.v_new,
                                self.centroids, self.cent_bf16, self.score_scale, self.sm_scale,
                                self.k, self.n_sink, self.n_local, self.mode, w.d_rand_u32,
                                self.scores, self.sel, self.k_out, self.sel_count, self.out,
                                self.lse, self.num_splits, self.workspace, self.workspace_bytes,
                                stream)

    def run_append(self, stream=None, one_call: bool = True) -> None:
        """An appending decode step: vx_append_decode_step, or (one_call =
        False) its two calls: the new token's K/V slot write and its page's
        centroid (append_kv), then the indexer and attention without a second
        refresh."""
        if self.indexer == "bounds":
            raise ValueError("the appending step is built for the centroid indexer")
        if one_call:
            self.append_step(stream)
            return
        self.append_kv(stream)
        self.step(refresh=False, stream=stream)

    def plan(self) -> dict:
        return V.vx_plan_decode(self.pages, self.geom, self.k_out, self.num_splits)

    def run(self, stream=None) -> None:
        """The whole step: cache refresh, scoring, selection, attention."""
        if self.indexer == "bounds":
            if self.fused:
                self.bound_step(stream=stream)
            else:
                self.bound_score(refresh=True, stream=stream)
                self.select(stream=stream)
                self.attend(stream=stream)
        elif self.fused:
            self.step(stream=stream)
        else:
            self.refresh_centroids(stream=stream)
            self.score(stream)
            self.select(stream=stream)
            self.attend(stream=stream)
