"""ctypes binding of libvx.so (include/vx.h): argument marshalling only.

Every computation runs in the library's gfx950 kernels. Tensors are torch
tensors used as device memory; the stream is torch's current stream unless
one is passed. Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_void_p
from typing import Optional

import torch

__all__ = [
    "VxError", "VxPages", "VxGeom", "VxPlan", "load", "lib_path", "status_string",
    "vx_centroid_update", "vx_page_scores", "vx_topk_pages", "vx_index_pages",
    "vx_sparse_decode", "vx_decode_step", "vx_plan_decode", "vx_check_pages", "vx_bounds_update",
    "vx_bound_scores", "vx_bound_decode_step", "vx_decode_step_static", "vx_append_decode_step", "VX_F32", "VX_BF16", "VX_TOPK_EXACT", "VX_TOPK_APPROX",
    "ENTRY_POINTS",
]

VX_OK, VX_ERR_INVALID_ARG, VX_ERR_UNSUPPORTED, VX_ERR_WORKSPACE, VX_ERR_HIP = range(5)
VX_F32, VX_BF16 = 0, 1
VX_TOPK_EXACT, VX_TOPK_APPROX = 0, 1
ENTRY_POINTS = ("vx_centroid_update", "vx_page_scores", "vx_topk_pages", "vx_index_pages",
                "vx_bounds_update", "vx_bound_scores", "vx_bound_decode_step",
                "vx_sparse_decode", "vx_decode_step", "vx_decode_step_static",
                "vx_append_decode_step", "vx_plan_decode", "vx_check_pages", "vx_status_string",
                "vx_last_error", "vx_abi_version")

_DTYPES = {torch.float32: VX_F32, torch.bfloat16: VX_BF16}


class VxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class VxPages(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("page_size", c_int32), ("num_pool_pages", c_int32),
                ("total_pages", c_int32), ("max_pages", c_int32), ("indptr", c_void_p),
                ("page_ids", c_void_p), ("seq_lens", c_void_p)]


class VxGeom(ctypes.Structure):
    _fields_ = [("num_q_heads", c_int32), ("num_kv_heads", c_int32), ("head_dim_k", c_int32),
                ("head_dim_v", c_int32), ("mla", c_int32), ("q_dtype", c_int32),
                ("kv_dtype", c_int32), ("score_dim", c_int32), ("score_bf16", c_int32)]


class VxPlan(ctypes.Structure):
    _fields_ = [("num_splits", c_int32), ("pages_per_split", c_int32),
                ("score_pages_per_block", c_int32), ("score_blocks", c_int32),
                ("topk_threads", c_int32), ("num_cus", c_int32), ("fused_step", c_int32),
                ("workspace_bytes", c_size_t), ("order_segments", c_int32),
                ("pair_segments", c_int32)]


_LIB: Optional[ctypes.CDLL] = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvx.so")


def load() -> ctypes.CDLL:
    """Load libvx.so from the package directory (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sparse_attention_decode_amd.build`")
    lib = ctypes.CDLL(path)
    P, G = POINTER(VxPages), POINTER(VxGeom)
    lib.vx_centroid_update.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p]
    lib.vx_page_scores.argtypes = [P, G, c_void_p, c_void_p, c_float, c_void_p, c_void_p]
    lib.vx_topk_pages.argtypes = [P, c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                  c_void_p, c_void_p, c_int32, c_void_p, c_void_p]
    lib.vx_index_pages.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                   c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                   c_void_p, c_int32, c_void_p, c_void_p]
    lib.vx_sparse_decode.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                     c_void_p, c_float, c_void_p, c_void_p, c_int32, c_void_p,
                                     POINTER(c_size_t), c_void_p]
    lib.vx_decode_step.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_float, c_float, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                   c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                   c_int32, c_void_p, POINTER(c_size_t), c_void_p]
    lib.vx_decode_step_static.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_int32, c_float, c_float, c_int32, c_int32,
                                          c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                          c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                          c_void_p]
    lib.vx_append_decode_step.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_float, c_float, c_int32, c_int32,
                                          c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                          c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                          POINTER(c_size_t), c_void_p]
    lib.vx_plan_decode.argtypes = [P, G, c_int32, c_int32, c_int32, POINTER(VxPlan)]
    lib.vx_check_pages.argtypes = [P, c_void_p, c_void_p]
    lib.vx_bounds_update.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.vx_bound_scores.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                    c_void_p, c_void_p]
    lib.vx_bound_decode_step.argtypes = [P, G, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                         c_float, c_float, c_int32, c_int32, c_int32, c_int32,
                                         c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                         c_void_p, c_void_p, c_int32, c_void_p,
                                         POINTER(c_size_t), c_void_p]
    for name in ("vx_centroid_update", "vx_page_scores", "vx_topk_pages", "vx_index_pages",
                 "vx_sparse_decode", "vx_decode_step", "vx_decode_step_static",
                 "vx_append_decode_step", "vx_plan_decode", "vx_bounds_update", "vx_bound_scores",
                 "vx_bound_decode_step", "vx_check_pages"):
        getattr(lib, name).restype = c_int32
    lib.vx_status_string.argtypes = [c_int32]
    lib.vx_status_string.restype = c_char_p
    lib.vx_last_error.argtypes = []
    lib.vx_last_error.restype = c_char_p
    lib.vx_abi_version.restype = c_int32
    _LIB = lib
    return lib


def status_string(st: int) -> str:
    return load().vx_status_string(st).decode()


def _check(st: int) -> None:
    if st != VX_OK:
        raise VxError(st, load().vx_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dt: torch.dtype) -> int:
    return _DTYPES[dt]


def make_pages(batch, page_size, num_pool_pages, total_pages, max_pages, indptr, page_ids,
               seq_lens) -> VxPages:
    return VxPages(batch, page_size, num_pool_pages, total_pages, max_pages, _ptr(indptr),
                   _ptr(page_ids), _ptr(seq_lens))


def make_geom(num_q_heads, num_kv_heads, head_dim_k, head_dim_v, mla, q_dtype, kv_dtype,
              score_dim: int = 0, score_bf16: bool = False) -> VxGeom:
    q = q_dtype if isinstance(q_dtype, int) else dtype_code(q_dtype)
    kv = kv_dtype if isinstance(kv_dtype, int) else dtype_code(kv_dtype)
    return VxGeom(num_q_heads, num_kv_heads, head_dim_k, head_dim_v, int(mla), q, kv,
                  int(score_dim), int(score_bf16))


def vx_centroid_update(pages: VxPages, geom: VxGeom, k_pool, v_pool, first_token, k_new, v_new,
                       centroids, cent_bf16, stream=None) -> None:
    _check(load().vx_centroid_update(ctypes.byref(pages), ctypes.byref(geom), _ptr(k_pool),
                                     _ptr(v_pool), _ptr(first_token), _ptr(k_new), _ptr(v_new),
                                     _ptr(centroids), _ptr(cent_bf16), _stream(stream)))


def vx_page_scores(pages: VxPages, geom: VxGeom, q, centroids, score_scale: float, scores,
                   stream=None) -> None:
    _check(load().vx_page_scores(ctypes.byref(pages), ctypes.byref(geom), _ptr(q),
                                 _ptr(centroids), float(score_scale), _ptr(scores),
                                 _stream(stream)))


def vx_bounds_update(pages: VxPages, geom: VxGeom, k_pool, first_token, bounds,
                     stream=None) -> None:
    _check(load().vx_bounds_update(ctypes.byref(pages), ctypes.byref(geom), _ptr(k_pool),
                                   _ptr(first_token), _ptr(bounds), _stream(stream)))


def vx_bound_scores(pages: VxPages, geom: VxGeom, q, k_pool, bounds, refresh_newest: bool,
                    score_scale: float, scores, stream=None) -> None:
    _check(load().vx_bound_scores(ctypes.byref(pages), ctypes.byref(geom), _ptr(q), _ptr(k_pool),
                                  _ptr(bounds), int(bool(refresh_newest)), float(score_scale),
                                  _ptr(scores), _stream(stream)))


def vx_topk_pages(pages: VxPages, num_kv_heads: int, scores, k: int, n_sink: int, n_local: int,
                  mode: int, rand_u32, sel, sel_stride: int, sel_count, stream=None) -> None:
    _check(load().vx_topk_pages(ctypes.byref(pages), num_kv_heads, _ptr(scores), k, n_sink,
                                n_local, mode, _ptr(rand_u32), _ptr(sel), sel_stride,
                                _ptr(sel_count), _stream(stream)))


def _nbytes(workspace, workspace_bytes) -> c_size_t:
    if workspace is not None and workspace_bytes is None:
        return c_size_t(workspace.numel() * workspace.element_size())
    return c_size_t(0 if workspace_bytes is None else workspace_bytes)


def vx_index_pages(pages: VxPages, geom: VxGeom, q, k_pool, centroids, cent_bf16,
                   refresh_newest: bool, score_scale: float, scores, k: int, n_sink: int,
                   n_local: int, mode: int, rand_u32, sel, sel_stride: int, sel_count,
                   stream=None) -> None:
    """Newest-page refresh (optional) + scores + top-k."""
    _check(load().vx_index_pages(ctypes.byref(pages), ctypes.byref(geom), _ptr(q), _ptr(k_pool),
                                 _ptr(centroids), _ptr(cent_bf16), int(refresh_newest),
                                 float(score_scale), _ptr(scores), k, n_sink, n_local, mode,
                                 _ptr(rand_u32), _ptr(sel), sel_stride, _ptr(sel_count),
                                 _stream(stream)))


def vx_sparse_decode(pages: VxPages, geom: VxGeom, q, k_pool, v_pool, sel, sel_stride: int,
                     sel_count, sm_scale: float, out, lse, num_splits: int = 0, workspace=None,
                     workspace_bytes: Optional[int] = None, stream=None) -> int:
    """Runs the attention; with workspace=None only returns the bytes needed."""
    nbytes = _nbytes(workspace, workspace_bytes)
    _check(load().vx_sparse_decode(ctypes.byref(pages), ctypes.byref(geom), _ptr(q), _ptr(k_pool),
                                   _ptr(v_pool), _ptr(sel), sel_stride, _ptr(sel_count),
                                   float(sm_scale), _ptr(out), _ptr(lse), num_splits,
                                   _ptr(workspace), ctypes.byref(nbytes), _stream(stream)))
    return nbytes.value


def vx_decode_step(pages: VxPages, geom: VxGeom, q, k_pool, v_pool, centroids, cent_bf16,
                   refresh_newest: bool, score_scale: float, sm_scale: float, k: int, n_sink: int,
                   n_local: int, mode: int, rand_u32, scores, sel, sel_stride: int, sel_count, out,
                   lse, num_splits: int = 0, workspace=None, workspace_bytes: Optional[int] = None,
                   stream=None) -> int:
    """Indexer + attention; with workspace=None only returns the bytes needed."""
    nbytes = _nbytes(workspace, workspace_bytes)
    _check(load().vx_decode_step(ctypes.byref(pages), ctypes.byref(geom), _ptr(q), _ptr(k_pool),
                                 _ptr(v_pool), _ptr(centroids), _ptr(cent_bf16),
                                 int(refresh_newest), float(score_scale), float(sm_scale), k,
                                 n_sink, n_local, mode, _ptr(rand_u32), _ptr(scores), _ptr(sel),
                                 sel_stride, _ptr(sel_count), _ptr(out), _ptr(lse), num_splits,
                                 _ptr(workspace), ctypes.byref(nbytes), _stream(stream)))
    return nbytes.value


def vx_append_decode_step(pages: VxPages, geom: VxGeom, q, k_pool, v_pool, k_new, v_new,
                          centroids, cent_bf16, score_scale: float, sm_scale: float, k: int,
                          n_sink: int, n_local: int, mode: int, rand_u32, scores, sel,
                          sel_stride: int, sel_count, out, lse, num_splits: int = 0,
                          workspace=None, workspace_bytes: Optional[int] = None,
                          stream=None) -> int:
    """Append of the newest token's K/V rows + the whole step; with workspace=None only
    returns the bytes needed."""
    nbytes = _nbytes(workspace, workspace_bytes)
    _check(load().vx_append_decode_step(ctypes.byref(pages), ctypes.byref(geom), _ptr(q),
                                        _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                                        _ptr(centroids), _ptr(cent_bf16), float(score_scale),
                                        float(sm_scale), k, n_sink, n_local, mode,
                                        _ptr(rand_u32), _ptr(scores), _ptr(sel), sel_stride,
                                        _ptr(sel_count), _ptr(out), _ptr(lse), num_splits,
                                        _ptr(workspace), ctypes.byref(nbytes), _stream(stream)))
    return nbytes.value


def vx_decode_step_static(pages: VxPages, geom: VxGeom, q, k_pool, v_pool, centroids, cent_bf16,
                          refresh_newest: bool, score_scale: float, sm_scale: float, k: int,
                          n_sink: int, n_local: int, mode: int, rand_u32, scores, sel,
                          sel_stride: int, sel_count, out, lse, num_splits: int = 0,
                          stream=None) -> None:
    """vx_decode_step with the library's own scratch (no workspace argument)."""
    _check(load().vx_decode_step_static(ctypes.byref(pages), ctypes.byref(geom), _ptr(q),
                                        _ptr(k_pool), _ptr(v_pool), _ptr(centroids),
                                        _ptr(cent_bf16), int(refresh_newest), float(score_scale),
                                        float(sm_scale), k, n_sink, n_local, mode,
                                        _ptr(rand_u32), _ptr(scores), _ptr(sel), sel_stride,
                                        _ptr(sel_count), _ptr(out), _ptr(lse), num_splits,
                                        _stream(stream)))


def vx_bound_decode_step(pages: VxPages, geom: VxGeom, q, k_pool, v_pool, bounds,
                         refresh_newest: bool, score_scale: float, sm_scale: float, k: int,
                         n_sink: int, n_local: int, mode: int, rand_u32, scores, sel,
                         sel_stride: int, sel_count, out, lse, num_splits: int = 0,
                         workspace=None, workspace_bytes: Optional[int] = None,
                         stream=None) -> int:
    """The whole step with the bounds indexer; with workspace=None only
    returns the bytes needed."""
    nbytes = _nbytes(workspace, workspace_bytes)
    _check(load().vx_bound_decode_step(ctypes.byref(pages), ctypes.byref(geom), _ptr(q),
                                       _ptr(k_pool), _ptr(v_pool), _ptr(bounds),
                                       int(refresh_newest), float(score_scale), float(sm_scale),
                                       k, n_sink, n_local, mode, _ptr(rand_u32), _ptr(scores),
                                       _ptr(sel), sel_stride, _ptr(sel_count), _ptr(out),
                                       _ptr(lse), num_splits, _ptr(workspace),
                                       ctypes.byref(nbytes), _stream(stream)))
    return nbytes.value


def vx_check_pages(pages: VxPages, counts, stream=None) -> None:
    """counts: device int32[3], written with the page table's contract
    violations (indptr order, sequence lengths, page ids out of the pool)."""
    _check(load().vx_check_pages(ctypes.byref(pages), _ptr(counts), _stream(stream)))


def vx_plan_decode(pages: VxPages, geom: VxGeom, sel_stride: int, num_splits: int = 0,
                   num_cus: int = 0) -> dict:
    plan = VxPlan()
    _check(load().vx_plan_decode(ctypes.byref(pages), ctypes.byref(geom), sel_stride, num_splits,
                                 num_cus, ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in VxPlan._fields_}
