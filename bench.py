#!/usr/bin/env python3
"""Benchmark of one block top-k sparse-attention decode step on one MI355X.

A step is the whole hot path over one batch: the indexer (cache-stage
refresh of each sequence's newest page, page scoring, top-k selection, fused
into one kernel where the shape allows) then split-K attention and its
log-sum-exp merge. Inputs are seeded synthetic tensors already resident
in HBM. Several replicas of the workload (same values, different memory)
rotate from step to step so that the 256 MB Infinity Cache cannot hold a
step's working set between two uses. Each step of a replica is captured once
in a HIP graph; the timed region replays them K times between two
synchronisations.

Prints one JSON line: seqs/s (value), KV tokens/s, achieved HBM GB/s of the
step and, in "roofline", of its dominant kernel stage (algorithmic bytes /
its average duration from HIP events around graph replays of that stage
alone), and "cpu_baseline", the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode seqs/s + KV tokens/s + achieved HBM GB/s vs peak"
PEAK_GBPS = 8000.0  # MI355X HBM3E
DESCR = {
    "tiny_fp32": "B=1 Hq=2 Hkv=1 D=64 P=16 L=1024 fp32, top-8 + last page",
    "gqa_bf16": "B=32 Hq=16 Hkv=8 D=128 P=16 L~U[2048,4096] bf16, top-16 + sink + last",
    "longgen_bf16": "B=64 Hq=32 Hkv=8 D=128 P=16 L~U[8192,32768] bf16, top-128 + sink + last 2",
    "mla_bf16": "B=32 Hq=32 latent 576 (512+64 rope) Dv=512 P=64 L~U[16384,65536] bf16, top-32 + sink + last",
    "largebatch_bf16": "B=256 Hq=64 Hkv=8 D=128 P=64 L~lognormal(16384, ln2) in [4096,65536] bf16, top-64",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa_bf16", choices=sorted(DESCR))
    ap.add_argument("--mode", default="exact", choices=["exact", "approx"])
    ap.add_argument("--indexer", default="centroid", choices=["centroid", "bounds"],
                    help="bounds: the Quest-style page-bounds indexer (GQA workloads)")
    ap.add_argument("--score-bf16", action="store_true",
                    help="GQA: score the pages on the centroids' bf16 copy (vx_geom.score_bf16)")
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to exceed 1 GB touched")
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="measure only --workload (by default the other workloads are measured "
                         "in the same run and reported under \"workloads\")")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy kernel (HBM counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="only write profiles/<workload>_step.md and profiles/traffic.json from "
                         "the rocprofv3 runs under DIR (see profile_commands)")
    ap.add_argument("--dense-compare", action="store_true",
                    help="sparse vs dense decode attention at a 32-query / 8-KV-head, D=128, "
                         "batch 16, 32K-token shape (prints its own JSON line)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(w, step):
    """Algorithmic bytes of one step: every in-use page's centroid row (or,
    for the bounds indexer, its min and max rows in the KV dtype) once, plus
    the valid tokens of every selected page (K and V rows)."""
    s = w.spec
    sel = step.sel.cpu().numpy()
    cnt = step.sel_count.cpu().numpy()
    P = s.page_size
    kv_elt = 4 if s.kv_dtype == "f32" else 2
    if step.indexer == "bounds":
        cent_elt = 2 * kv_elt
    else:  # MLA, and GQA with score_bf16, score the centroids' bf16 copy
        cent_elt = 2 if s.mla or getattr(step, "score_bf16", False) else 4
    n_pages = np.array([w.n_pages(b) for b in range(s.batch)])
    cent_bytes = int(n_pages.sum()) * s.num_kv_heads * s.head_dim_k * cent_elt
    row = (s.head_dim_k if s.mla else s.head_dim_k + s.head_dim_v) * kv_elt
    tokens = 0
    for b in range(s.batch):
        L = int(w.seq_lens[b])
        for g in range(s.num_kv_heads):
            ids = sel[b, g, :cnt[b, g]]
            tokens += int(np.clip(L - ids.astype(np.int64) * P, 0, P).sum())
    return cent_bytes, tokens * row, tokens


def refresh_bytes(w):
    """Keys of each sequence's newest page, read by the cache-stage refresh."""
    s = w.spec
    kv_elt = 4 if s.kv_dtype == "f32" else 2
    P = s.page_size
    nv = [(int(L) - 1) % P + 1 for L in w.seq_lens if L > 0]
    return int(sum(nv)) * s.num_kv_heads * s.head_dim_k * kv_elt


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_worker(args):
    """One CPU worker (a fresh process): the oracle's whole step over the
    sequences stored under `d`, round-robin from `first`, until `seconds`
    of work have run. Returns (sequence-steps, KV tokens attended, seconds)."""
    d, names, first, seconds, kw = args
    os.environ["OMP_NUM_THREADS"] = "1"
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, ROOT)
    from oracle import vx_oracle as O
    seqs = []
    for n in names:
        z = np.load(os.path.join(d, n + ".npz"))
        seqs.append({"q": z["q"].astype(np.float64), "k": z["k"].astype(np.float64),
                     "v": z["v"].astype(np.float64) if z["v"].size else None,
                     "seq_len": int(z["seq_len"]), "rand_u32": z["rand_u32"]})
    P, H = kw["page_size"], kw["num_kv_heads"]
    done, tokens, busy = 0, 0, 0.0
    with threadpool_limits(limits=1):
        i = first
        while busy < seconds:
            seq = seqs[i % len(seqs)]
            t0 = time.perf_counter()
            r = O.decode_sequence(seq, **kw)
            busy += time.perf_counter() - t0
            L = seq["seq_len"]
            ids = r["sel"][r["sel"] >= 0].astype(np.int64)
            tokens += int(np.clip(L - ids * P, 0, P).sum())
            done += 1
            i += 1
    return done, tokens / H, busy


def cpu_baseline(w, step, seconds):
    """The oracle as it stands (oracle/vx_oracle.py, numpy fp64) on the host
    cores, over whole sequences of the same workload: first one worker per
    host core the process may use (at most 16, the host share of one GPU),
    then a single worker, each for about `seconds` of work. Each
    sequence-step is the oracle's decode_sequence: it rebuilds the centroid
    of every page of the sequence (the GPU step refreshes only the newest
    page's), then scores, selects and attends."""
    import multiprocessing as mp
    import shutil
    import tempfile
    s = w.spec
    nseq = min(s.batch, 8)
    d = tempfile.mkdtemp(prefix="vx_cpu_")
    try:
        names = []
        for b in range(nseq):
            q = w.host_sequence(b)
            np.savez(os.path.join(d, f"s{b}.npz"), q=q["q"].astype(np.float32),
                     k=q["k"].astype(np.float32),
                     v=(q["v"].astype(np.float32) if q["v"] is not None else np.zeros(0)),
                     seq_len=q["seq_len"], rand_u32=q["rand_u32"])
            names.append(f"s{b}")
        kw = dict(page_size=s.page_size, num_kv_heads=s.num_kv_heads, k=step.k,
                  n_sink=step.n_sink, n_local=step.n_local, score_scale=step.score_scale,
                  sm_scale=step.sm_scale, mla=s.mla, head_dim_v=s.head_dim_v,
                  approx=step.mode == 1, indexer=step.indexer,
                  score_bf16=getattr(step, "score_bf16", False))
        cores = max(1, min(len(os.sched_getaffinity(0)), 16))
        ctx = mp.get_context("spawn")  # no fork of a process that holds the GPU
        res = {}
        for label, nw in (("all", cores), ("one", 1)):
            with ctx.Pool(nw) as pool:
                out = pool.map(_oracle_worker,
                               [(d, names, i, seconds, kw) for i in range(nw)])
            done = sum(o[0] for o in out)
            res[label] = {"seqs_per_s": sum(o[0] / o[2] for o in out),
                          "kv_tokens_per_s": sum(o[1] / o[2] for o in out),
                          "sequence_steps": done, "workers": nw}
    finally:
        shutil.rmtree(d, ignore_errors=True)
    one = res["one"]
    return {"value": res["all"]["seqs_per_s"], "unit": "seqs/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "kv_tokens_per_s": res["all"]["kv_tokens_per_s"],
            "one_core": {"value": one["seqs_per_s"], "unit": "seqs/s", "cores": 1,
                         "kv_tokens_per_s": one["kv_tokens_per_s"]},
            "sample": f"{res['all']['sequence_steps']} sequence-steps on {cores} worker processes "
                      f"(one numpy thread each, about {seconds:.0f} s of work per worker), then "
                      f"{one['sequence_steps']} on one, over the first {nseq} sequences of the same "
                      f"workload; each sequence-step is the oracle's whole step: the "
                      f"{'page bounds' if step.indexer == 'bounds' else 'centroids'} of every page "
                      f"rebuilt (the GPU step refreshes only the newest page's), then scores, "
                      f"selection and attention, in fp64"}


def sources_hash():
    """sha256 over the kernel sources with comments and blank lines removed:
    HBM traffic figures taken with other code no longer describe these
    kernels, while an edit of a comment leaves them valid."""
    import hashlib
    import re
    d = os.path.join(ROOT, "sparse_attention_decode_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            code = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
            h.update(name.encode())
            h.update(code.encode())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of a stage's kernels from profiles/traffic.json
    (rocprofv3 FETCH_SIZE and WRITE_SIZE passes, calibrated), or None when they
    were taken on other kernel sources or not at all."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get("workloads", {}).get(workload)
    if not e or e.get("sources_sha256") != sources_hash() or stage not in e.get("stages", {}):
        return None
    return e["stages"][stage]["hbm_bytes_per_launch"]


# Kernels whose HBM bytes make up each stage bench.py can report as dominant,
# per profiled run (workload, or workload + a suffix of RUN_VARIANTS).
PROFILE_STAGES = {
    "gqa_bf16": {"decode_step": ["decode_seg_kernel"], "indexer": ["index_seg_kernel"],
                 "attention_merge": ["attn_gqa_mfma_kernel"]},
    "largebatch_bf16": {"decode_step": ["decode_seg_kernel"], "indexer": ["index_seg_kernel"],
                        "attention_merge": ["attn_gqa_mfma_kernel"]},
    "longgen_bf16": {"decode_step": ["decode_seg_kernel"], "indexer": ["index_seg_kernel"],
                     "attention_merge": ["attn_gqa_mfma_kernel"]},
    "mla_bf16": {"indexer": ["scores_mla_kernel", "topk"],
                 "attention_merge": ["attn_mla_kernel", "merge_kernel"]},
    "tiny_fp32": {"decode_step": ["decode_seg_vec_kernel"], "indexer": ["index_seg_kernel"],
                  "attention_merge": ["attn_gqa_kernel"]},
    "gqa_bf16_bounds": {"decode_step": ["decode_seg_kernel"]},
    "largebatch_bf16_bounds": {"decode_step": ["decode_seg_kernel"]},
    "longgen_bf16_bounds": {"decode_step": ["decode_seg_kernel"]},
    "gqa_bf16_cb16": {"decode_step": ["decode_seg_kernel"]},
    "largebatch_bf16_cb16": {"decode_step": ["decode_seg_kernel"]},
    "longgen_bf16_cb16": {"decode_step": ["decode_seg_kernel"]},
}
# Run-name suffixes: the indexer variant and its bench.py flag.
RUN_VARIANTS = {"_bounds": "--indexer bounds", "_cb16": "--score-bf16"}
# The whole-step kernel's last two template arguments (bounds indexer, bf16
# centroid copy) for each variant.
STEP_KERNEL_TAIL = {"": "false, false>", "_bounds": "true, false>", "_cb16": "false, true>"}


def run_parts(run):
    """(workload, variant suffix, bench.py flags) of a profiled run name."""
    for suf, flag in RUN_VARIANTS.items():
        if run.endswith(suf):
            wl = run[:-len(suf)]
            return wl, suf, f"--workload {wl} {flag}"
    return run, "", f"--workload {run}"


def profile_commands(run):
    """The rocprofv3 runs a profiled run `run` (a PROFILE_STAGES key) needs,
    with their outputs under $OUT: a kernel trace, then one pass per HBM
    counter; the copy calibration passes run once for all."""
    _, _, flags = run_parts(run)
    cmds = [f"rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/{run}_trace -o run -- "
            f"python3 $R/bench.py {flags} --steps 50 --warmup 5 --stage-reps 5 --no-cpu-baseline --no-extras"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds.append(f"rocprofv3 --pmc {c} --kernel-trace --output-format csv -d $OUT/{run}_{c} -o run "
                    f"-- python3 $R/bench.py {flags} --steps 8 --warmup 2 --stage-reps 1 --no-cpu-baseline --no-extras")
    return cmds


def summarize_profiles(out, commit):
    """Writes profiles/<run>_step.md for every run profiled under `out` and
    profiles/traffic.json: per stage, the calibrated HBM bytes per launch
    (FETCH_SIZE and WRITE_SIZE scaled by what they read for a plain 1 GiB
    copy), keyed on sources_hash()."""
    import collections
    import csv
    import re
    import statistics

    def short(n):
        n = n.replace("(anonymous namespace)::", "").replace("void ", "").replace("vx::", "")
        return re.sub(r"\(.*", "", n).replace("unsigned short", "bf16")

    def durations(d):
        agg = collections.defaultdict(list)
        with open(os.path.join(d, "run_kernel_trace.csv")) as f:
            for r in csv.DictReader(f):
                agg[short(r["Kernel_Name"])].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        return agg

    def counters(d, name):
        agg = collections.defaultdict(list)
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == name:
                    agg[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return ({k: statistics.mean(v) for k, v in agg.items()}, {k: len(v) for k, v in agg.items()})

    cf, _ = counters(os.path.join(out, "copy_FETCH_SIZE"), "FETCH_SIZE")
    cw, _ = counters(os.path.join(out, "copy_WRITE_SIZE"), "WRITE_SIZE")
    copy_kernel = max(cf, key=lambda k: cf[k])
    kib = (1 << 30) / 1024
    ff, wf = kib / cf[copy_kernel], kib / cw[copy_kernel]
    sha = sources_hash()
    traffic = {"calibration": {"copy_kernel": copy_kernel, "bytes_read_and_written": 1 << 30,
                               "fetch_size_kib": cf[copy_kernel], "write_size_kib": cw[copy_kernel],
                               "fetch_factor": ff, "write_factor": wf},
               "commit_profiled": commit, "workloads": {}}
    for run, stages in PROFILE_STAGES.items():
        if not os.path.isdir(os.path.join(out, run + "_trace")):
            continue
        wl, suf, _ = run_parts(run)
        bounds = suf == "_bounds"
        dur = durations(os.path.join(out, run + "_trace"))
        fe, nf = counters(os.path.join(out, run + "_FETCH_SIZE"), "FETCH_SIZE")
        wr, _ = counters(os.path.join(out, run + "_WRITE_SIZE"), "WRITE_SIZE")
        with open(os.path.join(out, run + "_trace.log")) as f:
            text = f.read()
        tot, cent, kv = (float(x) for x in re.search(
            r"step touches ([\d.]+) MB \(centroids ([\d.]+), selected KV ([\d.]+)\)", text).groups())
        step_us = re.search(r"\d+ steps: ([\d.]+) us/step", text).group(1)
        stage_line = re.search(r"stage us: (.*)", text).group(1)
        title = {"": wl, "_bounds": f"{wl} with the Quest-style bounds indexer",
                 "_cb16": f"{wl} scoring the centroids' bf16 copy"}[suf]
        lines = [f"# {title}: one decode step, kernel durations and HBM traffic", "",
                 f"Profiled at commit `{commit}` on one MI355X. Algorithmic bytes per step: {tot:.1f} MB "
                 f"({'page bounds' if bounds else 'bf16 centroids' if suf else 'centroids'} "
                 f"{cent:.1f} MB + selected valid KV "
                 f"{kv:.1f} MB).", "",
                 "Commands (`cd /tmp && export TMPDIR=/tmp` first; `$R` = the repository, `$OUT` = the "
                 "output directory), then `python3 $R/bench.py --summarize-profiles $OUT`:", "", "```",
                 *profile_commands(run), "```", "",
                 f"Same-run bench (under the profiler): {step_us} us/step; stages (each alone) "
                 f"{stage_line}.", "",
                 "| kernel | dispatches | mean us | median us | min us | FETCH_SIZE KiB | WRITE_SIZE KiB "
                 "| HBM MB (calibrated) |", "|---|---|---|---|---|---|---|---|"]
        for k, v in sorted(dur.items(), key=lambda kv_: -statistics.mean(kv_[1]) * len(kv_[1])):
            if not k.startswith(("decode_seg", "decode_mla", "index_", "attn_", "merge", "scores_",
                                 "topk", "centroid_", "bound")):
                continue
            f_, w_ = fe.get(k), wr.get(k)
            hb = "" if f_ is None or w_ is None else round((f_ * ff + w_ * wf) * 1024 / 1e6, 2)
            lines.append(f"| `{k}` | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} "
                         f"| {min(v):.2f} | {f_ if f_ is None else round(f_, 1)} | "
                         f"{w_ if w_ is None else round(w_, 1)} | {hb} |")
        entry = {"sources_sha256": sha, "stages": {}}
        for st, pats in stages.items():
            parts, total = [], 0.0
            for pat in pats:
                match = [k for k in fe if pat in k and (not pat.startswith("decode_seg")
                                                        or k.endswith(STEP_KERNEL_TAIL[suf]))]
                if not match:
                    raise SystemExit(f"{run}: no counters for {pat}")
                k = max(match, key=lambda x: nf[x])  # the stage's instantiation: most dispatches
                b = (fe[k] * ff + wr.get(k, 0.0) * wf) * 1024
                total += b
                parts.append({"kernel": k, "fetch_size_kib": fe[k], "write_size_kib": wr.get(k, 0.0),
                              "hbm_bytes": b})
            entry["stages"][st] = {"kernels": parts, "hbm_bytes_per_launch": total}
        traffic["workloads"][run] = entry
        lines += ["", f"Calibration (`bench.py --copy-calibration`, a torch elementwise copy reading and "
                      f"writing 1 GiB): FETCH_SIZE {cf[copy_kernel]:.1f} KiB and WRITE_SIZE "
                      f"{cw[copy_kernel]:.1f} KiB per dispatch, so FETCH_SIZE is scaled by {ff:.3f} and "
                      f"WRITE_SIZE by {wf:.3f}.", "",
                  "HBM bytes per launch of the stages bench.py can report as dominant:", ""]
        for st, e in entry["stages"].items():
            lines.append(f"- `{st}`: {e['hbm_bytes_per_launch'] / 1e6:.2f} MB "
                         f"({', '.join(p_['kernel'] for p_ in e['kernels'])})")
        mf = os.path.join(out, run + "_MFMA")
        if os.path.isdir(mf):
            vals = collections.defaultdict(lambda: collections.defaultdict(list))
            with open(os.path.join(mf, "run_counter_collection.csv")) as f:
                for r in csv.DictReader(f):
                    vals[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
            mdur = durations(mf)
            lines += ["", "## MFMA use (MLA kernels)", "", "```",
                      f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAVE_CYCLES "
                      f"SQ_INSTS_MFMA --kernel-trace --output-format csv -d $OUT/{run}_MFMA -o run -- "
                      f"python3 $R/bench.py --workload {wl} --steps 8 --warmup 2 --stage-reps 1 "
                      f"--no-cpu-baseline --no-extras", "```", "",
                      "| kernel | mean us (under counters) | SQ_INSTS_MFMA | SQ_VALU_MFMA_BUSY_CYCLES "
                      "| SQ_BUSY_CU_CYCLES | MFMA busy / CU busy |", "|---|---|---|---|---|---|"]
            for k in sorted(vals):
                if not k.startswith(("scores_mla", "attn_mla", "decode_mla")):
                    continue
                v = {c: statistics.mean(x) for c, x in vals[k].items()}
                busy, cu = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), v.get("SQ_BUSY_CU_CYCLES", 0.0)
                lines.append(f"| `{k}` | {statistics.mean(mdur[k]):.2f} | {v.get('SQ_INSTS_MFMA', 0):.0f} "
                             f"| {busy:.0f} | {cu:.0f} | {100 * busy / cu if cu else 0:.1f} % |")
            lines += ["", "By flops the scorer's [32 x 576] x [576 x pages] contraction is about 0.76 "
                          "GFLOP per step and the", "attention's q.k^T and P.V about 9.7 GFLOP (32 heads "
                          "x 2176 tokens x (576 + 512) x 2 x 32", "sequences); both read far more bytes "
                          "per flop than the matrix cores' ridge, so HBM and",
                      "latency bound them, and the MFMA busy fraction stays low."]
        with open(os.path.join(ROOT, "profiles", f"{run}_step.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"wrote profiles/{run}_step.md")
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    log("wrote profiles/traffic.json")


def overlap(w, step, sel_a, cnt_a, sel_b, cnt_b):
    """Mean and minimum over (sequence, KV head) of |A ∩ B| / min(k, candidates),
    forced pages excluded: the recall@k of selection A against selection B."""
    s = w.spec
    a, ca = sel_a.cpu().numpy(), cnt_a.cpu().numpy()
    e, ce = sel_b.cpu().numpy(), cnt_b.cpu().numpy()
    rec = []
    for b in range(s.batch):
        n = w.n_pages(b)
        forced = set(range(min(n, step.n_sink))) | set(range(max(0, n - step.n_local), n))
        want = min(step.k, n - len(forced))
        if want <= 0:
            continue
        for g in range(s.num_kv_heads):
            sa = set(a[b, g, :ca[b, g]].tolist()) - forced
            se = set(e[b, g, :ce[b, g]].tolist()) - forced
            rec.append(len(sa & se) / want)
    return {"mean": float(np.mean(rec)), "min": float(np.min(rec)), "segments": len(rec)}


def approx_recall(w, step):
    """recall@k of the approximate selection against the exact one on the
    same scores."""
    import torch
    from sparse_attention_decode_amd import binding as V
    s = w.spec
    sel_e = torch.full_like(step.sel, -1)
    cnt_e = torch.zeros_like(step.sel_count)
    V.vx_topk_pages(step.pages, s.num_kv_heads, step.scores, step.k, step.n_sink, step.n_local,
                    V.VX_TOPK_EXACT, None, sel_e, step.k_out, cnt_e)
    torch.cuda.synchronize()
    return overlap(w, step, step.sel, step.sel_count, sel_e, cnt_e)


def rope_unaware_recall(w, step):
    """MLA: recall@k of the selection scored on the 512 latent columns only
    against the rope-aware selection (all 576 columns)."""
    import torch
    from sparse_attention_decode_amd.step import DecodeStep
    alt = DecodeStep(w, score_dim=512)
    alt.rebuild_centroids()
    alt.index(refresh=False)
    torch.cuda.synchronize()
    return overlap(w, step, alt.sel, alt.sel_count, step.sel, step.sel_count)


def attention_mass(w, step):
    """Mean and minimum over (sequence, query head) of the share of the head's
    full softmax weight (over every valid token) that falls on the pages
    selected for its KV head: how much of dense attention the selection keeps.
    A quality report, computed with plain fp32 torch ops on the GPU."""
    import torch
    s = w.spec
    P, Hkv, D = s.page_size, s.num_kv_heads, s.head_dim_k
    G = s.num_q_heads // Hkv
    sel, cnt = step.sel.cpu().numpy(), step.sel_count.cpu().numpy()
    masses = []
    for b in range(s.batch):
        L, n = int(w.seq_lens[b]), w.n_pages(b)
        if L == 0:
            continue
        lo = int(w.indptr[b])
        ids = torch.from_numpy(w.page_ids[lo:lo + n].astype(np.int64)).to(w.device)
        k = w.k_pool.index_select(0, ids).float()[..., :D]          # [n][Hkv][P][D]
        k = k.permute(1, 0, 2, 3).reshape(Hkv, n * P, D)            # [Hkv][nP][D]
        kt = k.transpose(1, 2).contiguous()
        q = w.q[b].float()[:, :D].reshape(Hkv, G, D).contiguous()
        z = torch.matmul(q, kt) * step.sm_scale                       # [Hkv][G][nP]
        z[..., L:] = float("-inf")
        pm = torch.softmax(z, dim=-1).reshape(Hkv, G, n, P).sum(-1)  # [Hkv][G][n]
        for g in range(Hkv):
            chosen = torch.from_numpy(sel[b, g, :cnt[b, g]].astype(np.int64)).to(w.device)
            masses.append(pm[g].index_select(1, chosen).sum(-1).cpu())
    m = torch.cat(masses)
    return {"mean": float(m.mean()), "min": float(m.min()), "heads": int(m.numel())}


def copy_calibration():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log("copy calibration: 5 launches, each reads 1 GiB and writes 1 GiB")


def stream_copy_GBps():
    """Bytes moved per second by a plain device copy of 1 GiB (1 GiB read +
    1 GiB written), the streaming rate this machine reaches, reported next to
    the step's rate."""
    import torch
    n = 1 << 28
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 5 * 2 * (n * 4) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def dense_compare(a):
    """Decode attention over the selected pages vs over every page (k = all
    pages, the same kernels), at a shape like the pages' kernel ablation:
    32 query / 8 KV heads, D = 128, batch 16, 32K tokens; budget top-128 +
    sink + last 2 pages (the long-generation workload's)."""
    import torch
    from sparse_attention_decode_amd import workloads as W
    from sparse_attention_decode_amd.step import DecodeStep
    sp = W.spec("longgen_bf16", batch=16, lengths=("fixed", 32768), headroom_tokens=0)
    log("dense compare: generating B=16 x 32768 tokens")
    w = W.make(sp, "cuda", seed=0)
    sparse = DecodeStep(w)
    dense = DecodeStep(w, k=w.max_pages, n_sink=0, n_local=0)
    for st in (sparse, dense):
        st.rebuild_centroids()
        st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def timed(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream, capture_error_mode="thread_local"):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            g.replay()
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    t_sparse_attn = timed(sparse.attend, 50)
    t_sparse_step = timed(sparse.run, 50)
    t_dense_attn = timed(dense.attend, 20)
    _, kv_s, tok_s = step_bytes(w, sparse)
    _, kv_d, tok_d = step_bytes(w, dense)
    res = {"metric": "decode attention us: sparse (selected pages) vs dense (every page)",
           "value": t_dense_attn / t_sparse_attn, "unit": "x (dense / sparse attention time)",
           "n_gpus": 1, "higher_is_better": True, "data": "synthetic", "dtype": "bf16",
           "config": {"workload": "B=16 Hq=32 Hkv=8 D=128 P=16 L=32768 bf16; sparse budget "
                                  "top-128 + sink + last 2 pages"},
           "sparse_attention_us": t_sparse_attn, "sparse_step_us": t_sparse_step,
           "dense_attention_us": t_dense_attn, "sparse_kv_bytes": kv_s, "dense_kv_bytes": kv_d,
           "sparse_attention_GBps": kv_s / t_sparse_attn / 1e3,
           "dense_attention_GBps": kv_d / t_dense_attn / 1e3,
           "pages_context": "the pages' kernel ablation: sparse 0.025 ms vs dense 0.760 ms "
                            "(Qwen3-8B, batch 16, 32K, hardware unstated)"}
    print(json.dumps(res), flush=True)


# The workload each default run also measures beside the headline one, so
# every configuration's step is timed in the same run; the long-generation
# workload's step appends a token (K/V slot write + that page's centroid),
# and the two large ones also report the indexer in exact and approximate
# top-k mode.
# The largest workload first: its 27 GB of pools, allocated after the other
# workloads' pools have been freed, ran 3-5 % slower (the same kernels, a
# different physical placement of the pools).
EXTRA_WORKLOADS = ("largebatch_bf16", "mla_bf16", "longgen_bf16", "tiny_fp32")
APPEND_WORKLOADS = ("longgen_bf16",)
INDEX_MODE_WORKLOADS = ("longgen_bf16", "largebatch_bf16")


class Bench:
    """The replicas of one workload, their step graphs and timings."""

    def __init__(self, name, mode, indexer, replicas, append, score_bf16=False):
        import torch
        from sparse_attention_decode_amd import workloads as W
        from sparse_attention_decode_amd.step import DecodeStep
        self.name, self.mode, self.indexer, self.append = name, mode, indexer, append
        self.score_bf16 = score_bf16
        sp = W.spec(name)
        self.spec = sp
        log(f"workload {name}: generating on cuda:0")
        w0 = W.make(sp, "cuda", seed=0)
        base = DecodeStep(w0, mode=mode, indexer=indexer, score_bf16=score_bf16)
        base.rebuild()
        self.run_fn = (lambda st: st.run_append()) if append else (lambda st: st.run())
        self.run_fn(base)
        torch.cuda.synchronize()
        self.w0, self.base = w0, base
        self.cent_b, self.kv_b, self.tokens = step_bytes(w0, base)
        self.plan = base.plan()
        total = self.cent_b + self.kv_b
        self.R = replicas or max(1, min(16, math.ceil(1.0e9 / total)))
        log(f"step touches {total / 1e6:.1f} MB (centroids {self.cent_b / 1e6:.1f}, selected KV "
            f"{self.kv_b / 1e6:.1f}); {self.R} replica(s)")
        self.ws, self.steps = [w0], [base]
        for _ in range(self.R - 1):
            w = w0.replicate()
            st = DecodeStep(w, mode=mode, indexer=indexer, score_bf16=score_bf16)
            st.rebuild()
            self.ws.append(w)
            self.steps.append(st)
        torch.cuda.synchronize()
        self.stream = torch.cuda.Stream()
        self.stream.wait_stream(torch.cuda.current_stream())

    def capture(self, fn):
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            for st in self.steps:  # one eager pass before capture
                fn(st)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=self.stream, capture_error_mode="thread_local"):
            for st in self.steps:
                fn(st)
        torch.cuda.synchronize()
        return g

    def time_step(self, steps, warmup):
        """us per step over `steps` steps (graph replays of all replicas, then
        single-replica graphs for the remainder), timed with HIP events on
        the replay stream between two synchronisations."""
        import torch
        g_step = self.capture(self.run_fn)
        singles = []
        for st in self.steps:
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=self.stream, capture_error_mode="thread_local"):
                self.run_fn(st)
            singles.append(g1)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            for _ in range(max(1, warmup // self.R)):
                g_step.replay()
        torch.cuda.synchronize()
        full, rem = divmod(steps, self.R)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.stream):
            ev0.record(self.stream)
            for _ in range(full):
                g_step.replay()
            for i in range(rem):
                singles[i].replay()
            ev1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us = ev0.elapsed_time(ev1) * 1e3 / steps
        log(f"{self.name}: {steps} steps: {us:.2f} us/step (host wall {wall * 1e6 / steps:.2f} us)")
        return us

    def time_stage(self, fn, reps):
        """us per call of fn (graph replays of every replica, HIP events on the
        replay stream)."""
        import torch
        g = self.capture(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            g.replay()
            e0.record(self.stream)
            for _ in range(reps):
                g.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * self.R)

    def stages(self, full):
        """The stage functions to time: every stage for the headline workload,
        otherwise those the roofline needs."""
        if self.indexer == "bounds":
            st = {"decode_step": lambda x: x.bound_step(),
                  "indexer": lambda x: (x.bound_score(refresh=True), x.select()),
                  "attention_merge": lambda x: x.attend()}
            if full:
                st.update({"cache_refresh": lambda x: x.refresh_bounds(),
                           "page_scores": lambda x: x.bound_score(),
                           "bound_scores_refresh": lambda x: x.bound_score(refresh=True),
                           "topk": lambda x: x.select()})
            return st
        refresh = not self.append
        st = {"decode_step": lambda x: x.step(refresh=refresh),
              "indexer": lambda x: x.index(refresh=refresh),
              "attention_merge": lambda x: x.attend()}
        if self.append:
            st["append_kv"] = lambda x: x.append_kv()
        if full:
            st.update({"cache_refresh": lambda x: x.refresh_centroids(),
                       "page_scores": lambda x: x.score(),
                       "topk": lambda x: x.select()})
        return st

    def record(self, a, full):
        """One workload's measurements: the step, its stages and the roofline
        of its dominant kernel stage."""
        us = self.time_step(a.steps, a.warmup)
        stage_us = {k: self.time_stage(fn, a.stage_reps) for k, fn in self.stages(full).items()}
        log(f"{self.name}: stage us: " + ", ".join(f"{k} {v:.2f}" for k, v in stage_us.items()))
        s = self.spec
        t_step = us * 1e-6
        total = self.cent_b + self.kv_b
        ref_b = 0 if self.append else refresh_bytes(self.w0)
        stage_bytes = {"decode_step": self.cent_b + ref_b + self.kv_b,
                       "indexer": self.cent_b + ref_b, "page_scores": self.cent_b,
                       "bound_scores_refresh": self.cent_b + refresh_bytes(self.w0),
                       "attention_merge": self.kv_b}
        stage_bytes = {k: v for k, v in stage_bytes.items() if k in stage_us}
        # One kernel per step when the plan fuses it; otherwise the indexer and
        # the attention (+ merge) run in turn and the slower is dominant.
        if self.plan["fused_step"]:
            dom = "decode_step"
        else:
            dom = max(("indexer", "attention_merge"), key=lambda k: stage_us[k])
        achieved = stage_bytes[dom] / (stage_us[dom] * 1e-6) / 1e9
        run = self.name + ("_bounds" if self.indexer == "bounds" else
                           "_cb16" if self.score_bf16 else "")
        rec = {"workload": f"{self.name}: {DESCR[self.name]}",
               "ms_per_step": us / 1e3, "seqs_per_s": s.batch / t_step,
               "kv_tokens_per_s": self.tokens / s.num_kv_heads / t_step,
               "step_bytes": total, "step_hbm_GBps": total / t_step / 1e9,
               "step_frac_of_peak": total / t_step / 1e9 / PEAK_GBPS,
               "replicas": self.R, "num_splits": self.plan["num_splits"],
               "fused_step": bool(self.plan["fused_step"]), "appends_token": self.append,
               "stage_us": stage_us,
               "stage_GBps": {k: stage_bytes[k] / (stage_us[k] * 1e-6) / 1e9 for k in stage_bytes},
               "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS,
                            "unit": "GB/s", "frac": achieved / PEAK_GBPS,
                            "traffic": measured_traffic(run, dom), "kernel": dom,
                            "bytes_per_launch": stage_bytes[dom]}}
        return rec

    def free(self):
        import torch
        del self.steps, self.ws, self.base, self.w0
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def bf16_copy_scoring(b, a):
    """The same workload and replicas with the pages scored on the
    centroids' bf16 copy (GQA, vx_geom.score_bf16): the step's time, bytes
    and rate, and the recall@k of its selection against the fp32-centroid
    selection of the same step on the same inputs."""
    import torch
    from sparse_attention_decode_amd.step import DecodeStep
    fp32, alt = b.steps, []
    for w in b.ws:
        st = DecodeStep(w, mode=b.mode, score_bf16=True)
        st.rebuild()
        alt.append(st)
    b.steps = alt
    try:
        us = b.time_step(a.steps, a.warmup)
        dec = b.time_stage(lambda x: x.step(refresh=not b.append), a.stage_reps)
    finally:
        b.steps = fp32
    b.base.step(refresh=True)
    alt[0].step(refresh=True)
    torch.cuda.synchronize()
    rec = overlap(b.w0, b.base, alt[0].sel, alt[0].sel_count, b.base.sel, b.base.sel_count)
    cent_b, kv_b, _ = step_bytes(b.w0, alt[0])
    del alt
    torch.cuda.empty_cache()
    s = b.spec
    out = {"ms_per_step": us / 1e3, "seqs_per_s": s.batch / (us * 1e-6),
           "step_bytes": cent_b + kv_b, "centroid_bytes": cent_b,
           "step_hbm_GBps": (cent_b + kv_b) / (us * 1e-6) / 1e9,
           "decode_step_us": dec, "recall_at_k_vs_fp32_centroids": rec}
    log(f"{b.name} scoring the bf16 centroid copy: {us:.2f} us/step, decode_step {dec:.2f} us, "
        f"recall@k vs fp32 centroids mean {rec['mean']:.4f} min {rec['min']:.4f}")
    return out


# GQA bf16 workloads that also report bf16-copy scoring in the default run.
BF16_COPY_WORKLOADS = ("gqa_bf16", "longgen_bf16", "largebatch_bf16")


def index_modes(name, a):
    """The indexer stage (vx_index_pages) in exact and in approximate top-k
    mode on the same workload, with the approximate selection's recall@k
    against the exact one on the same scores."""
    from sparse_attention_decode_amd import binding as V
    out = {}
    for label, mode in (("exact", V.VX_TOPK_EXACT), ("approx", V.VX_TOPK_APPROX)):
        b = Bench(name, mode, "centroid", a.replicas, False)
        out[f"indexer_us_{label}"] = b.time_stage(lambda x: x.index(), a.stage_reps)
        out[f"topk_us_{label}"] = b.time_stage(lambda x: x.select(), a.stage_reps)
        if mode == V.VX_TOPK_APPROX:
            out["approx_recall_at_k"] = approx_recall(b.w0, b.base)
        b.free()
    out["indexer_speedup_approx"] = out["indexer_us_exact"] / out["indexer_us_approx"]
    out["topk_speedup_approx"] = out["topk_us_exact"] / out["topk_us_approx"]
    log(f"{name}: indexer exact {out['indexer_us_exact']:.2f} us, approx "
        f"{out['indexer_us_approx']:.2f} us; top-k alone {out['topk_us_exact']:.2f} / "
        f"{out['topk_us_approx']:.2f} us; recall@k {out['approx_recall_at_k']['mean']:.4f}")
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              f"(the path shards by sequence with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if a.summarize_profiles:
        import subprocess
        commit = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"],
                                capture_output=True, text=True).stdout.strip() or "unknown"
        summarize_profiles(a.summarize_profiles, os.environ.get("PROFILED_COMMIT") or commit)
        return
    if a.copy_calibration:
        copy_calibration()
        return
    if a.dense_compare:
        dense_compare(a)
        return

    from sparse_attention_decode_amd import binding as V

    torch.cuda.set_device(0)
    mode = V.VX_TOPK_APPROX if a.mode == "approx" else V.VX_TOPK_EXACT
    from sparse_attention_decode_amd import workloads as W
    sp = W.spec(a.workload)
    bounds = a.indexer == "bounds"
    if bounds and sp.mla:
        print("the bounds indexer is implemented for GQA workloads only", file=sys.stderr)
        sys.exit(2)
    append = a.workload in APPEND_WORKLOADS and not bounds
    if a.score_bf16 and (sp.mla or bounds or sp.kv_dtype != "bf16"):
        print("--score-bf16 applies to the centroid indexer of bf16 GQA workloads",
              file=sys.stderr)
        sys.exit(2)
    main_b = Bench(a.workload, mode, a.indexer, a.replicas, append, a.score_bf16)
    w0, base = main_b.w0, main_b.base
    recall = approx_recall(w0, base) if mode == V.VX_TOPK_APPROX else None
    if recall:
        log(f"approximate top-k recall@k: mean {recall['mean']:.4f}, min {recall['min']:.4f} "
            f"over {recall['segments']} segments")
    rope = rope_unaware_recall(w0, base) if sp.mla and mode == V.VX_TOPK_EXACT else None
    if rope:
        log(f"rope-unaware MLA selection vs rope-aware, recall@k: mean {rope['mean']:.4f}, "
            f"min {rope['min']:.4f}")
    quality = None
    if bounds:
        from sparse_attention_decode_amd.step import DecodeStep
        cent = DecodeStep(w0, mode=mode)
        cent.rebuild()
        cent.run()
        torch.cuda.synchronize()
        quality = {"attention_mass_bounds": attention_mass(w0, base),
                   "attention_mass_centroid": attention_mass(w0, cent),
                   "overlap_with_centroid": overlap(w0, base, base.sel, base.sel_count,
                                                    cent.sel, cent.sel_count)}
        log("selected share of dense softmax weight: bounds "
            f"{quality['attention_mass_bounds']['mean']:.4f}, centroid "
            f"{quality['attention_mass_centroid']['mean']:.4f}; selection overlap "
            f"{quality['overlap_with_centroid']['mean']:.4f}")
        del cent
    rec = main_b.record(a, full=True)
    copy_gbps = stream_copy_GBps()
    log(f"streaming copy of 1 GiB: {copy_gbps:.0f} GB/s (read + write)")
    s = sp
    result = {
        "metric": METRIC,
        "value": rec["seqs_per_s"],
        "unit": "seqs/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if s.kv_dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": rec["workload"], "topk_mode": a.mode,
                   "indexer": a.indexer + (" (bf16 copy)" if a.score_bf16 else ""),
                   "replicas": rec["replicas"], "hip_graph": True,
                   "num_splits": rec["num_splits"], "fused_step": rec["fused_step"],
                   "appends_token": rec["appends_token"]},
        "kv_tokens_per_s": rec["kv_tokens_per_s"],
        "step_bytes": rec["step_bytes"],
        "step_hbm_GBps": rec["step_hbm_GBps"],
        "step_frac_of_peak": rec["step_frac_of_peak"],
        "stream_copy_GBps": copy_gbps,
        "stage_us": rec["stage_us"],
        "stage_GBps": rec["stage_GBps"],
        "roofline": rec["roofline"],
    }
    if recall:
        result["approx_recall_at_k"] = recall
    if rope:
        result["mla_rope_unaware_recall_at_k"] = rope
    if quality:
        result["selection_quality"] = quality
    if not a.no_extras and not bounds and mode == V.VX_TOPK_EXACT:
        if a.workload in BF16_COPY_WORKLOADS and not a.score_bf16:
            result["bf16_centroid_scoring"] = bf16_copy_scoring(main_b, a)
        # The other workloads, each measured in this same run.
        main_b.free()
        result["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            if name == a.workload:
                continue
            b = Bench(name, mode, "centroid", a.replicas, name in APPEND_WORKLOADS)
            r = b.record(a, full=False)
            if name in BF16_COPY_WORKLOADS:
                r["bf16_centroid_scoring"] = bf16_copy_scoring(b, a)
            b.free()
            if name in INDEX_MODE_WORKLOADS:
                r["topk_modes"] = index_modes(name, a)
            result["workloads"][name] = r
        # the headline workload's CPU baseline needs its inputs again
        main_b = None
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        if main_b is None:
            main_b = Bench(a.workload, mode, a.indexer, 1, append, a.score_bf16)
        result["cpu_baseline"] = cpu_baseline(main_b.w0, main_b.base, a.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
