"""Builds libvx.so (the gfx950 kernels and their C ABI) in-tree with hipcc.

Each source compiles to its own object in parallel (the kernels of one file
are launched only from that file, so no relocatable device code is needed),
then one hipcc link makes the shared library.

Usage: python -m sparse_attention_decode_amd.build   (or build() from Python)
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libvx.so")
SOURCES = ["vx_capi.hip", "centroid.hip", "scores.hip", "indexer.hip", "topk.hip", "attention.hip",
           "mla.hip", "decode.hip", "bounds.hip", "pages.hip"]
ARCH = "gfx950"
# no packed fp32 instructions in generated code
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return res.returncode, out


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source for gfx950 and link libvx.so next to this file."""
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(OBJ, s + ".o") for s in SOURCES]
    cmds = [[cc, *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or max(1, min(len(cmds), len(os.sched_getaffinity(0)), 16))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
