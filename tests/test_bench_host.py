"""Host logic of bench.py (no GPU): the algorithmic byte count, the
selection overlap (recall@k), and the source hash that keys the HBM traffic
table (comments do not change it, code does)."""

import importlib.util
import os
import shutil
from types import SimpleNamespace

import numpy as np
import torch

from sparse_attention_decode_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def small_workload():
    sp = W.spec("gqa_bf16", batch=2, num_q_heads=4, num_kv_heads=2,
                lengths=("list", (40, 17)))  # pages 3 (last holds 8) and 2 (last holds 1)
    return W.make(sp, "cpu", seed=3)


def fake_step(w, sel, indexer="centroid", k=2, n_sink=0, n_local=1):
    sel = torch.tensor(sel, dtype=torch.int32)
    cnt = (sel >= 0).sum(-1).to(torch.int32)
    return SimpleNamespace(sel=sel, sel_count=cnt, indexer=indexer, k=k, n_sink=n_sink,
                           n_local=n_local)


def test_step_bytes_counts_valid_tokens_and_index_rows():
    B = load_bench()
    w = small_workload()
    # sequence 0 selects pages 0 and 2 (16 + 8 tokens), sequence 1 page 1 (1 token), per KV head
    step = fake_step(w, [[[0, 2, -1], [0, 2, -1]], [[1, -1, -1], [1, -1, -1]]])
    cent, kv, tokens = B.step_bytes(w, step)
    assert tokens == 2 * (16 + 8) + 2 * 1
    assert kv == tokens * (128 + 128) * 2
    assert cent == (3 + 2) * 2 * 128 * 4  # fp32 centroid rows of every page in use
    bcent, _, _ = B.step_bytes(w, fake_step(w, step.sel.tolist(), indexer="bounds"))
    assert bcent == (3 + 2) * 2 * 128 * 2 * 2  # bf16 minima and maxima


def test_overlap_is_recall_without_forced_pages():
    B = load_bench()
    w = small_workload()
    a = fake_step(w, [[[0, 1, 2], [0, 1, 2]], [[0, 1, -1], [0, 1, -1]]])
    same = B.overlap(w, a, a.sel, a.sel_count, a.sel, a.sel_count)
    assert same["mean"] == 1.0 and same["min"] == 1.0
    # sequence 0: forced = last page (2); candidates 0, 1 both wanted (k = 2); the other
    # selection keeps page 0 only -> recall 1/2 on both heads; sequence 1: 1 candidate
    b = fake_step(w, [[[0, 2, -1], [0, 2, -1]], [[0, 1, -1], [0, 1, -1]]])
    r = B.overlap(w, a, b.sel, b.sel_count, a.sel, a.sel_count)
    assert r["min"] == 0.5 and np.isclose(r["mean"], (0.5 + 0.5 + 1 + 1) / 4)


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    B = load_bench()
    src = os.path.join(ROOT, "sparse_attention_decode_amd", "csrc")
    copy = tmp_path / "sparse_attention_decode_amd" / "csrc"
    shutil.copytree(src, copy, ignore=shutil.ignore_patterns("*.o", "*.hipfb"))
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    h0 = B.sources_hash()
    f = copy / "bounds.h"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("#pragma once", "#pragma once  /* x */"))
    assert B.sources_hash() == h0
    f.write_text(text + "\nconstexpr int vx_extra = 1;\n")
    assert B.sources_hash() != h0


def test_measured_traffic_unknown_workload_is_none():
    B = load_bench()
    assert B.measured_traffic("no_such_workload", "decode_step") is None


def _csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_summarize_profiles_calibrates_counters(tmp_path, monkeypatch):
    """Counters of a synthetic profiled run: FETCH_SIZE is scaled by what it
    reads for the 1 GiB copy (here half of it: factor 2), WRITE_SIZE likewise
    (factor 1); the stage's bytes per launch are the scaled sum."""
    B = load_bench()
    out = tmp_path / "prof"
    copy = "void at::native::copy_kernel(float)"
    kern = "void vx::(anonymous namespace)::decode_seg_kernel<2, 16, 16, false, false>(vx::SegArgs)"
    cc = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _csv(str(out / "copy_FETCH_SIZE" / "run_counter_collection.csv"), cc,
         [[f'"{copy}"', "FETCH_SIZE", 524288.0]])
    _csv(str(out / "copy_WRITE_SIZE" / "run_counter_collection.csv"), cc,
         [[f'"{copy}"', "WRITE_SIZE", 1048576.0]])
    _csv(str(out / "gqa_bf16_FETCH_SIZE" / "run_counter_collection.csv"), cc,
         [[f'"{kern}"', "FETCH_SIZE", 1000.0], [f'"{kern}"', "FETCH_SIZE", 1000.0]])
    _csv(str(out / "gqa_bf16_WRITE_SIZE" / "run_counter_collection.csv"), cc,
         [[f'"{kern}"', "WRITE_SIZE", 10.0]])
    _csv(str(out / "gqa_bf16_trace" / "run_kernel_trace.csv"),
         ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
         [[f'"{kern}"', 1000, 19000], [f'"{kern}"', 50000, 68000]])
    with open(out / "gqa_bf16_trace.log", "w") as f:
        f.write("[bench] step touches 62.4 MB (centroids 25.7, selected KV 36.7); 16 replica(s)\n"
                "[bench] 50 steps: 18.50 us/step (host wall 18.70 us)\n"
                "[bench] stage us: decode_step 18.20\n")
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    monkeypatch.setattr(B, "sources_hash", lambda: "h")
    monkeypatch.setattr(B, "PROFILE_STAGES", {"gqa_bf16": {"decode_step": ["decode_seg_kernel"]}})
    B.summarize_profiles(str(out), "abc1234")
    import json
    t = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert t["calibration"]["fetch_factor"] == 2.0 and t["calibration"]["write_factor"] == 1.0
    st = t["workloads"]["gqa_bf16"]["stages"]["decode_step"]
    assert st["hbm_bytes_per_launch"] == (1000.0 * 2 + 10.0) * 1024
    md = (tmp_path / "profiles" / "gqa_bf16_step.md").read_text()
    assert "| `decode_seg_kernel<2, 16, 16, false, false>` | 2 | 18.00 |" in md
    assert "abc1234" in md


def test_run_names_map_to_bench_flags():
    """A profiled run's name gives its workload, variant and bench.py flags."""
    import bench as B
    assert B.run_parts("gqa_bf16") == ("gqa_bf16", "", "--workload gqa_bf16")
    assert B.run_parts("longgen_bf16_bounds") == ("longgen_bf16", "_bounds",
                                                  "--workload longgen_bf16 --indexer bounds")
    assert B.run_parts("largebatch_bf16_cb16") == ("largebatch_bf16", "_cb16",
                                                   "--workload largebatch_bf16 --score-bf16")
    assert set(B.STEP_KERNEL_TAIL) == {""} | set(B.RUN_VARIANTS)


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so,
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
