"""The boundary is a C ABI: a plain C program that includes only
include/sp24.h and links libsp24.so compiles with gcc -std=c99 and passes
its host-side checks (no device needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")


def test_plain_c_client(tmp_path):
    from structured_sparse_transformer_amd import sp24
    if not os.path.exists(sp24.LIB_PATH):
        from structured_sparse_transformer_amd import build
        build.build()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(sp24.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), SRC, "-o", str(exe),
           "-L", libdir, "-l:libsp24.so", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
