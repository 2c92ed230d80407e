"""The boundary is a C ABI: include/swr.h compiles as C99 and a C program
linked against libswr.so calls the host-only layout planner (no GPU)."""
import os
import shutil
import subprocess

import pytest

import sharded_weight_reassembly_amd as swr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_program_uses_the_header_and_library(tmp_path):
    lib_dir = os.path.dirname(swr.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    # the HIP runtime header needs its platform named when a plain C compiler reads it
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I",
           os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", lib_dir, "-lswr", f"-Wl,-rpath,{lib_dir}",
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "c abi ok" in out.stdout
