"""include/vx.h from plain C: tests/c/abi_from_c.c compiles with gcc as C11
against the header, links libvx.so and runs its host-side checks (no GPU)."""

import os
import shutil
import subprocess

import pytest

from sparse_attention_decode_amd import binding as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs gcc and the ROCm headers")
def test_header_is_c_and_library_links(tmp_path):
    lib_dir = os.path.dirname(V.lib_path())
    assert os.path.exists(V.lib_path()), "build libvx.so first"
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L" + lib_dir, "-lvx",
           "-Wl,-rpath," + lib_dir, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
