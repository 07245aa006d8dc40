"""Host-side checks of libvx.so: it loads, exports every symbol include/vx.h
declares, rejects bad arguments before any HIP call, and plans launches.
No GPU is needed: nothing here launches a kernel."""

import ctypes
import os
import re

import pytest

from sparse_attention_decode_amd import binding as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAD = 0x1000  # never dereferenced: every call below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "vx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vx_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = V.load()
    names = header_functions()
    assert set(V.ENTRY_POINTS) <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.vx_abi_version() == 8


def pages(batch=2, page_size=16, pool=10, nnz=8, maxp=4, ptrs=True):
    p = BAD if ptrs else None
    return V.make_pages(batch, page_size, pool, nnz, maxp, p, p, p)


def geom(hq=16, hkv=8, dk=128, dv=128, mla=0, qd=V.VX_BF16, kvd=V.VX_BF16, score_dim=0,
         score_bf16=0):
    return V.make_geom(hq, hkv, dk, dv, mla, qd, kvd, score_dim, score_bf16)


def status_of(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except V.VxError as e:
        return e.status
    return V.VX_OK


def test_status_strings():
    assert V.status_string(0) == "VX_OK"
    assert V.status_string(3) == "VX_ERR_WORKSPACE"
    assert V.status_string(99) == "VX_ERR_UNKNOWN"


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=32), V.VX_ERR_UNSUPPORTED),
    (dict(batch=-1), V.VX_ERR_INVALID_ARG),
    (dict(maxp=9), V.VX_ERR_INVALID_ARG),
    (dict(ptrs=False), V.VX_ERR_INVALID_ARG),
    (dict(pool=0), V.VX_ERR_INVALID_ARG),
])
def test_bad_pages_rejected(kw, status):
    assert status_of(V.vx_page_scores, pages(**kw), geom(), BAD, BAD, 1.0, BAD, stream=0) == status
    assert status_of(V.vx_centroid_update, pages(**kw), geom(), BAD, None, None, None, None, BAD,
                     None, stream=0) == status


@pytest.mark.parametrize("kw,status", [
    (dict(hq=12, hkv=8), V.VX_ERR_INVALID_ARG),
    (dict(dk=96, dv=96), V.VX_ERR_UNSUPPORTED),
    (dict(dk=128, dv=64), V.VX_ERR_UNSUPPORTED),
    (dict(qd=V.VX_F32), V.VX_ERR_UNSUPPORTED),
    (dict(hkv=2, mla=1, dk=576, dv=512, hq=32), V.VX_ERR_INVALID_ARG),
    (dict(hkv=1, mla=1, dk=512, dv=512, hq=32), V.VX_ERR_UNSUPPORTED),
    (dict(hkv=32, hq=32, dk=128, dv=128), V.VX_ERR_UNSUPPORTED),  # 32*128 > 2048
    (dict(score_dim=64), V.VX_ERR_UNSUPPORTED),  # GQA scores every column
    (dict(hkv=1, mla=1, dk=576, dv=512, hq=32, score_dim=500), V.VX_ERR_UNSUPPORTED),
    (dict(score_bf16=2), V.VX_ERR_INVALID_ARG),
    (dict(score_bf16=1, qd=V.VX_F32, kvd=V.VX_F32), V.VX_ERR_UNSUPPORTED),  # bf16 KV only
])
def test_bad_geometry_rejected(kw, status):
    assert status_of(V.vx_page_scores, pages(), geom(**kw), BAD, BAD, 1.0, BAD, stream=0) == status


def test_topk_argument_checks():
    p = pages()
    ok = dict(k=4, n_sink=1, n_local=1, mode=0, rand_u32=None, sel=BAD, sel_stride=6, sel_count=BAD)

    def call(**kw):
        a = dict(ok, **kw)
        return status_of(V.vx_topk_pages, p, 8, BAD, a["k"], a["n_sink"], a["n_local"], a["mode"],
                         a["rand_u32"], a["sel"], a["sel_stride"], a["sel_count"], stream=0)

    assert call(sel_stride=5) == V.VX_ERR_INVALID_ARG
    assert call(k=-1) == V.VX_ERR_INVALID_ARG
    assert call(mode=2) == V.VX_ERR_INVALID_ARG
    assert call(mode=1) == V.VX_ERR_INVALID_ARG  # approx without random words
    assert call(sel=None) == V.VX_ERR_INVALID_ARG
    big = V.make_pages(1, 16, 20000, 17000, 17000, BAD, BAD, BAD)
    assert status_of(V.vx_topk_pages, big, 1, BAD, 4, 0, 0, 0, None, BAD, 4, BAD,
                     stream=0) == V.VX_ERR_UNSUPPORTED


def test_centroid_argument_checks():
    p, g = pages(), geom()
    # k_new needs the append mode
    assert status_of(V.vx_centroid_update, p, g, BAD, None, None, BAD, None, BAD, None,
                     stream=0) == V.VX_ERR_INVALID_ARG
    # v_new needs v_pool
    assert status_of(V.vx_centroid_update, p, g, BAD, None, BAD, BAD, BAD, BAD, None,
                     stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_centroid_update, p, g, BAD, None, None, None, None, None, None,
                     stream=0) == V.VX_ERR_INVALID_ARG
    # score_bf16: the cache stage keeps the bf16 copy
    assert status_of(V.vx_centroid_update, p, geom(score_bf16=1), BAD, None, None, None, None,
                     BAD, None, stream=0) == V.VX_ERR_INVALID_ARG


def test_decode_argument_checks():
    p = pages()
    # group of 3 query heads per KV head is not a supported attention geometry
    assert status_of(V.vx_sparse_decode, p, geom(hq=24, hkv=8), BAD, BAD, BAD, BAD, 4, BAD, 1.0,
                     BAD, None, 0, BAD, 1 << 20, stream=0) == V.VX_ERR_UNSUPPORTED
    assert status_of(V.vx_sparse_decode, p, geom(), BAD, BAD, BAD, BAD, 0, BAD, 1.0,
                     BAD, None, 0, BAD, 1 << 20, stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_sparse_decode, p, geom(), BAD, BAD, BAD, BAD, 4, BAD, float("nan"),
                     BAD, None, 0, BAD, 1 << 20, stream=0) == V.VX_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op():
    p = V.make_pages(0, 16, 0, 0, 0, None, None, None)
    V.vx_page_scores(p, geom(), None, None, 1.0, None, stream=0)
    V.vx_topk_pages(p, 8, None, 4, 1, 1, 0, None, None, 6, None, stream=0)
    V.vx_centroid_update(p, geom(), None, None, None, None, None, BAD, None, stream=0)


def test_planner_splits_and_workspace():
    g = geom()
    # 32 sequences x 8 KV heads already give one block per compute unit: no split
    plan = V.vx_plan_decode(pages(batch=32, nnz=6144, pool=7680, maxp=256), g, 18, 0, 256)
    assert plan["num_splits"] == 1 and plan["workspace_bytes"] == 0
    # a small batch is split so that about one block runs per compute unit, each split
    # streaming at least 128 KB: 18 pages x 64 tokens x 512 B = 576 KB -> 4 splits
    plan = V.vx_plan_decode(pages(batch=2, nnz=40, pool=40, maxp=20, page_size=64), g, 18, 0, 256)
    S, pps = plan["num_splits"], plan["pages_per_split"]
    assert S == 4 and pps == 5
    assert plan["workspace_bytes"] >= 2 * 16 * S * (128 + 2) * 4
    # 18 pages x 16 tokens x 512 B = 144 KB: one split, no merge
    plan = V.vx_plan_decode(pages(batch=2, nnz=40, pool=40, maxp=20), g, 18, 0, 256)
    assert plan["num_splits"] == 1 and plan["workspace_bytes"] == 0
    # an explicit split count is honoured (balanced splits, largest one reported)
    plan = V.vx_plan_decode(pages(batch=2, nnz=40, pool=40, maxp=20), g, 18, 7, 256)
    assert plan["num_splits"] == 7 and plan["pages_per_split"] == 3
    # never more splits than selected pages, never more than 256 pages per split
    tiny = g.__class__(2, 1, 64, 64, 0, 0, 0)
    plan = V.vx_plan_decode(pages(batch=1, nnz=64, pool=128, maxp=64), tiny, 9, 50, 256)
    assert plan["num_splits"] == 9
    # 9 pages x 16 tokens x 512 B (fp32, D = 64) = 72 KB: one split
    plan = V.vx_plan_decode(pages(batch=1, nnz=64, pool=128, maxp=64), tiny, 9, 0, 256)
    assert plan["num_splits"] == 1
    # at 64-token pages 288 KB: two splits
    plan = V.vx_plan_decode(pages(batch=1, nnz=64, pool=128, maxp=64, page_size=64), tiny, 9, 0, 256)
    assert plan["num_splits"] == 2
    plan = V.vx_plan_decode(pages(batch=4096, nnz=500000, pool=500000, maxp=200), g, 131, 1, 256)
    assert plan["pages_per_split"] == 131 and plan["num_splits"] == 1
    plan = V.vx_plan_decode(pages(batch=4096, nnz=500000, pool=500000, maxp=300), g, 260, 1, 256)
    assert plan["pages_per_split"] <= 256 and plan["num_splits"] == 2
    plan = V.vx_plan_decode(pages(batch=4096, nnz=2000000, pool=2000000, maxp=600), g, 520, 1, 256)
    assert plan["pages_per_split"] <= 256 and plan["num_splits"] == 3
    # MLA: one block per sequence and split
    mla = V.make_geom(32, 1, 576, 512, 1, V.VX_BF16, V.VX_BF16)
    plan = V.vx_plan_decode(pages(batch=32, nnz=20480, pool=25600, maxp=1024, page_size=64), mla, 34, 0, 256)
    assert plan["num_splits"] == 7 and plan["pages_per_split"] == 5  # 8 splits would also take 5


def test_planner_orders_long_batches():
    """Sequence lengths are device data, so the planner's length-dependent part
    runs on the device: when the whole step's segments span more than two
    rounds of blocks it asks vx_decode_step to rank the sequences longest first,
    and the step's workspace grows by 4 bytes per sequence."""
    g = geom(hq=64, hkv=8)
    # the large-batch shape: 256 sequences x 8 KV heads = 2048 segments > 2 x 256
    big = pages(batch=256, nnz=81600, pool=102000, maxp=1024, page_size=64)
    plan = V.vx_plan_decode(big, g, 64, 0, 256)
    assert plan["fused_step"] == 1 and plan["order_segments"] == 1
    assert plan["workspace_bytes"] == 0  # vx_decode_step adds 256 x 4 bytes for the order
    assert plan["pair_segments"] == 0
    # every block resident from the start, two 8-wave blocks per compute unit
    # (the long-generation shape, 512 segments on 256): no ranking launch, no
    # workspace; the step kernel pairs 32 rows of long sequences with the rest
    plan = V.vx_plan_decode(pages(batch=64, nnz=81920, pool=102400, maxp=2052), geom(hq=32), 131,
                            0, 256)
    assert plan["fused_step"] == 1 and plan["order_segments"] == 0
    assert plan["pair_segments"] == 32 and plan["workspace_bytes"] == 0
    # one block per compute unit (256 segments), or 16-wave blocks: not paired
    plan = V.vx_plan_decode(pages(batch=32, nnz=6144, pool=7680, maxp=256), geom(), 18, 0, 256)
    assert plan["fused_step"] == 1 and plan["pair_segments"] == 0
    plan = V.vx_plan_decode(pages(batch=48, nnz=9216, pool=11520, maxp=256), geom(), 18, 0, 256)
    assert plan["fused_step"] == 1 and plan["pair_segments"] == 0
    # split plans are not whole-step kernels: never ordered
    plan = V.vx_plan_decode(big, g, 64, 3, 256)
    assert plan["order_segments"] == 0
    # beyond the largest ordered batch
    plan = V.vx_plan_decode(pages(batch=2048, nnz=2048 * 20, pool=2048 * 25, maxp=20), g, 18, 0, 256)
    assert plan["order_segments"] == 0


def test_index_pages_argument_checks():
    p, g = pages(), geom()
    ok = dict(q=BAD, k_pool=BAD, centroids=BAD, cent_bf16=None, refresh=1, scale=1.0, scores=BAD,
              k=4, n_sink=1, n_local=1, mode=0, rand_u32=None, sel=BAD, stride=6, count=BAD,
              pages=p, geom=g)

    def call(**kw):
        a = dict(ok, **kw)
        return status_of(V.vx_index_pages, a["pages"], a["geom"], a["q"], a["k_pool"],
                         a["centroids"], a["cent_bf16"], a["refresh"], a["scale"], a["scores"],
                         a["k"], a["n_sink"], a["n_local"], a["mode"], a["rand_u32"], a["sel"],
                         a["stride"], a["count"], stream=0)

    assert call(refresh=2) == V.VX_ERR_INVALID_ARG
    assert call(scale=float("inf")) == V.VX_ERR_INVALID_ARG
    assert call(stride=5) == V.VX_ERR_INVALID_ARG
    assert call(k=-1) == V.VX_ERR_INVALID_ARG
    assert call(mode=1) == V.VX_ERR_INVALID_ARG  # approx without random words
    assert call(k_pool=None) == V.VX_ERR_INVALID_ARG  # refresh reads the keys
    assert call(centroids=None) == V.VX_ERR_INVALID_ARG
    assert call(q=None) == V.VX_ERR_INVALID_ARG
    assert call(sel=None) == V.VX_ERR_INVALID_ARG
    assert call(scores=None) == V.VX_ERR_INVALID_ARG
    mla = V.make_geom(32, 1, 576, 512, 1, V.VX_BF16, V.VX_BF16)
    mp = pages(page_size=64)
    assert call(geom=mla, pages=mp) == V.VX_ERR_INVALID_ARG  # MLA scores cent_bf16
    assert call(geom=geom(score_bf16=1)) == V.VX_ERR_INVALID_ARG  # so does score_bf16
    assert call(geom=geom(dk=96, dv=96)) == V.VX_ERR_UNSUPPORTED
    assert call(pages=pages(page_size=32)) == V.VX_ERR_UNSUPPORTED
    big = V.make_pages(1, 16, 20000, 17000, 17000, BAD, BAD, BAD)
    assert call(pages=big) == V.VX_ERR_UNSUPPORTED
    # an empty batch launches nothing
    e = V.make_pages(0, 16, 0, 0, 0, None, None, None)
    assert call(pages=e, q=None, k_pool=None, centroids=None, scores=None, sel=None,
                count=None) == V.VX_OK


def test_decode_step_argument_checks():
    p, g = pages(), geom()
    ok = dict(q=BAD, k_pool=BAD, v_pool=BAD, centroids=BAD, cent_bf16=None, refresh=1, sscale=1.0,
              smscale=1.0, k=4, n_sink=1, n_local=1, mode=0, rand_u32=None, scores=BAD, sel=BAD,
              stride=6, count=BAD, out=BAD, lse=None, splits=0, ws=BAD, ws_bytes=1 << 30,
              pages=p, geom=g)

    def call(**kw):
        a = dict(ok, **kw)
        return status_of(V.vx_decode_step, a["pages"], a["geom"], a["q"], a["k_pool"], a["v_pool"],
                         a["centroids"], a["cent_bf16"], a["refresh"], a["sscale"], a["smscale"],
                         a["k"], a["n_sink"], a["n_local"], a["mode"], a["rand_u32"], a["scores"],
                         a["sel"], a["stride"], a["count"], a["out"], a["lse"], a["splits"],
                         a["ws"], a["ws_bytes"], stream=0)

    assert call(refresh=2) == V.VX_ERR_INVALID_ARG
    assert call(sscale=float("nan")) == V.VX_ERR_INVALID_ARG
    assert call(smscale=float("inf")) == V.VX_ERR_INVALID_ARG
    assert call(stride=5) == V.VX_ERR_INVALID_ARG
    assert call(mode=1) == V.VX_ERR_INVALID_ARG
    assert call(v_pool=None) == V.VX_ERR_INVALID_ARG
    assert call(out=None) == V.VX_ERR_INVALID_ARG
    assert call(scores=None) == V.VX_ERR_INVALID_ARG
    assert call(centroids=None) == V.VX_ERR_INVALID_ARG
    assert call(geom=geom(score_bf16=1)) == V.VX_ERR_INVALID_ARG  # scores need cent_bf16
    assert call(geom=geom(hq=24, hkv=8)) == V.VX_ERR_UNSUPPORTED
    assert call(pages=pages(page_size=32)) == V.VX_ERR_UNSUPPORTED


def test_static_decode_step_argument_checks():
    """vx_decode_step_static runs vx_decode_step's checks before any HIP call
    (it has no workspace to query or check)."""
    p, g = pages(), geom()
    ok = dict(q=BAD, k_pool=BAD, v_pool=BAD, centroids=BAD, cent_bf16=None, refresh=1, sscale=1.0,
              smscale=1.0, k=4, n_sink=1, n_local=1, mode=0, rand_u32=None, scores=BAD, sel=BAD,
              stride=6, count=BAD, out=BAD, lse=None, splits=0, pages=p, geom=g)

    def call(**kw):
        a = dict(ok, **kw)
        return status_of(V.vx_decode_step_static, a["pages"], a["geom"], a["q"], a["k_pool"],
                         a["v_pool"], a["centroids"], a["cent_bf16"], a["refresh"], a["sscale"],
                         a["smscale"], a["k"], a["n_sink"], a["n_local"], a["mode"],
                         a["rand_u32"], a["scores"], a["sel"], a["stride"], a["count"], a["out"],
                         a["lse"], a["splits"], stream=0)

    assert call(refresh=2) == V.VX_ERR_INVALID_ARG
    assert call(sscale=float("nan")) == V.VX_ERR_INVALID_ARG
    assert call(stride=5) == V.VX_ERR_INVALID_ARG
    assert call(mode=1) == V.VX_ERR_INVALID_ARG
    assert call(v_pool=None) == V.VX_ERR_INVALID_ARG
    assert call(out=None) == V.VX_ERR_INVALID_ARG
    assert call(scores=None) == V.VX_ERR_INVALID_ARG
    assert call(geom=geom(hq=24, hkv=8)) == V.VX_ERR_UNSUPPORTED
    assert call(pages=pages(page_size=32)) == V.VX_ERR_UNSUPPORTED


def test_plan_reports_the_whole_step_kernel():
    g = geom()
    big = pages(batch=32, nnz=6144, pool=7680, maxp=256)
    assert V.vx_plan_decode(big, g, 18, 0, 256)["fused_step"] == 1
    assert V.vx_plan_decode(big, g, 18, 2, 256)["fused_step"] == 0  # two splits
    assert V.vx_plan_decode(big, g, 131, 0, 256)["fused_step"] == 1
    assert V.vx_plan_decode(big, g, 257, 0, 256)["fused_step"] == 0  # selection > 256 pages
    assert V.vx_plan_decode(big, geom(qd=V.VX_F32, kvd=V.VX_F32), 18, 0, 256)["fused_step"] == 1
    assert V.vx_plan_decode(big, geom(dk=64, dv=64), 18, 0, 256)["fused_step"] == 1
    assert V.vx_plan_decode(big, geom(hq=24, hkv=8), 18, 0, 256)["fused_step"] == 0  # group of 3
    huge = pages(batch=32, nnz=200000, pool=200000, maxp=5000)
    assert V.vx_plan_decode(huge, g, 18, 0, 256)["fused_step"] == 0  # capacity > 4096 pages
    small = pages(batch=2, nnz=40, pool=40, maxp=20, page_size=64)
    assert V.vx_plan_decode(small, g, 18, 0, 256)["fused_step"] == 0  # planner splits
    assert V.vx_plan_decode(small, g, 18, 1, 256)["fused_step"] == 1
    # 144 KB per selection at 16-token pages: too little to split, one kernel
    assert V.vx_plan_decode(pages(batch=2, nnz=40, pool=40, maxp=20), g, 18, 0, 256)["fused_step"] == 1


def test_bounds_argument_checks():
    """The Quest-style cache stage and scorer: GQA only, pointers and flags
    checked on the host before any launch; an empty batch is a no-op."""
    p, g = pages(), geom()
    mla = geom(hkv=1, mla=1, dk=576, dv=512, hq=32)
    assert status_of(V.vx_bounds_update, p, mla, BAD, None, BAD, stream=0) == V.VX_ERR_UNSUPPORTED
    assert status_of(V.vx_bound_scores, p, mla, BAD, BAD, BAD, True, 1.0, BAD,
                     stream=0) == V.VX_ERR_UNSUPPORTED
    assert status_of(V.vx_bounds_update, p, g, None, None, BAD, stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_bounds_update, p, g, BAD, None, None, stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_bounds_update, pages(page_size=32), g, BAD, None, BAD,
                     stream=0) == V.VX_ERR_UNSUPPORTED
    assert status_of(V.vx_bound_scores, p, geom(dk=96, dv=96), BAD, BAD, BAD, False, 1.0, BAD,
                     stream=0) == V.VX_ERR_UNSUPPORTED
    # refresh needs the key pool; scores and bounds are required; the scale finite
    assert status_of(V.vx_bound_scores, p, g, BAD, None, BAD, True, 1.0, BAD,
                     stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_bound_scores, p, g, BAD, None, None, False, 1.0, BAD,
                     stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_bound_scores, p, g, BAD, None, BAD, False, 1.0, None,
                     stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_bound_scores, p, g, None, None, BAD, False, 1.0, BAD,
                     stream=0) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_bound_scores, p, g, BAD, None, BAD, False, float("inf"), BAD,
                     stream=0) == V.VX_ERR_INVALID_ARG
    lib = V.load()
    st = lib.vx_bound_scores(ctypes.byref(p), ctypes.byref(g), BAD, BAD, BAD, 2, 1.0, BAD, None)
    assert st == V.VX_ERR_INVALID_ARG
    empty = V.make_pages(0, 16, 0, 0, 0, None, None, None)
    V.vx_bounds_update(empty, g, None, None, None, stream=0)
    V.vx_bound_scores(empty, g, None, None, None, True, 1.0, None, stream=0)


def test_bound_decode_step_argument_checks():
    p, g = pages(), geom()
    ok = dict(q=BAD, k_pool=BAD, v_pool=BAD, bounds=BAD, refresh=1, sscale=1.0, smscale=1.0,
              k=4, n_sink=1, n_local=1, mode=0, rand_u32=None, scores=BAD, sel=BAD, stride=6,
              count=BAD, out=BAD, lse=None, splits=0, ws=BAD, ws_bytes=1 << 30, pages=p, geom=g)

    def call(**kw):
        a = dict(ok, **kw)
        return status_of(V.vx_bound_decode_step, a["pages"], a["geom"], a["q"], a["k_pool"],
                         a["v_pool"], a["bounds"], a["refresh"], a["sscale"], a["smscale"],
                         a["k"], a["n_sink"], a["n_local"], a["mode"], a["rand_u32"], a["scores"],
                         a["sel"], a["stride"], a["count"], a["out"], a["lse"], a["splits"],
                         a["ws"], a["ws_bytes"], stream=0)

    assert call(geom=geom(hkv=1, mla=1, dk=576, dv=512, hq=32)) == V.VX_ERR_UNSUPPORTED
    assert call(refresh=2) == V.VX_ERR_INVALID_ARG
    assert call(sscale=float("nan")) == V.VX_ERR_INVALID_ARG
    assert call(smscale=float("inf")) == V.VX_ERR_INVALID_ARG
    assert call(stride=5) == V.VX_ERR_INVALID_ARG
    assert call(mode=1) == V.VX_ERR_INVALID_ARG
    assert call(v_pool=None) == V.VX_ERR_INVALID_ARG
    assert call(out=None) == V.VX_ERR_INVALID_ARG
    assert call(scores=None) == V.VX_ERR_INVALID_ARG
    assert call(bounds=None) == V.VX_ERR_INVALID_ARG
    assert call(geom=geom(hq=24, hkv=8)) == V.VX_ERR_UNSUPPORTED
    assert call(pages=pages(page_size=32)) == V.VX_ERR_UNSUPPORTED


def test_append_decode_step_argument_checks():
    """vx_append_decode_step: vx_decode_step's checks plus the new token's
    rows (k_new always, v_new without MLA, none with MLA), all before any HIP
    call."""
    p, g = pages(), geom()
    ok = dict(q=BAD, k_pool=BAD, v_pool=BAD, k_new=BAD, v_new=BAD, centroids=BAD, cent_bf16=None,
              sscale=1.0, smscale=1.0, k=4, n_sink=1, n_local=1, mode=0, rand_u32=None,
              scores=BAD, sel=BAD, stride=6, count=BAD, out=BAD, lse=None, splits=0, pages=p,
              geom=g)

    def call(**kw):
        a = dict(ok, **kw)
        return status_of(V.vx_append_decode_step, a["pages"], a["geom"], a["q"], a["k_pool"],
                         a["v_pool"], a["k_new"], a["v_new"], a["centroids"], a["cent_bf16"],
                         a["sscale"], a["smscale"], a["k"], a["n_sink"], a["n_local"], a["mode"],
                         a["rand_u32"], a["scores"], a["sel"], a["stride"], a["count"], a["out"],
                         a["lse"], a["splits"], workspace=BAD, workspace_bytes=1 << 30, stream=0)

    assert call(k_new=None) == V.VX_ERR_INVALID_ARG
    assert call(v_new=None) == V.VX_ERR_INVALID_ARG
    mla = geom(hq=32, hkv=1, dk=576, dv=512, mla=1)
    assert call(geom=mla, v_pool=None) == V.VX_ERR_INVALID_ARG  # v_new given with MLA
    assert call(sscale=float("nan")) == V.VX_ERR_INVALID_ARG
    assert call(stride=5) == V.VX_ERR_INVALID_ARG
    assert call(out=None) == V.VX_ERR_INVALID_ARG
    assert call(geom=geom(hq=24, hkv=8)) == V.VX_ERR_UNSUPPORTED


def test_check_pages_argument_checks():
    counts = BAD
    assert status_of(V.vx_check_pages, pages(), None) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_check_pages, pages(page_size=32), counts) == V.VX_ERR_UNSUPPORTED
    assert status_of(V.vx_check_pages, pages(ptrs=False), counts) == V.VX_ERR_INVALID_ARG
    assert status_of(V.vx_check_pages, pages(maxp=9), counts) == V.VX_ERR_INVALID_ARG
