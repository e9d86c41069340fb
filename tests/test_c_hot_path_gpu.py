"""The hot path driven from plain C.

tests/c_abi/hot_path.c includes only include/sp24.h and the HIP runtime's C
API. It allocates with hipMalloc and runs sp24_search_compress,
sp24_spmm_fwd and sp24_spmm_bwd_input on the null stream, with no Python or
torch in its process. Its outputs must equal the oracle's: bit for bit for
the masks and both 2:4 forms, and within the GEMM tolerance for the
products. The client is built by __graft_entry__.build() (gcc, host code
only), or here if that binary is missing.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

from forms_layout import block_width, from_blocked

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "hot_path.c")
PREBUILT = os.path.join(ROOT, "tests", "c_abi", "hot_path")
MAX_REL, MEAN_ABS = 1e-2, 1e-3


def client(tmp_path):
    if os.path.exists(PREBUILT) and os.path.getmtime(PREBUILT) >= os.path.getmtime(SRC):
        return PREBUILT
    from structured_sparse_transformer_amd import sp24
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available to build the C client")
    exe = str(tmp_path / "hot_path")
    subprocess.run(compile_command(gcc, exe, os.path.dirname(sp24.LIB_PATH)), check=True, capture_output=True,
                   text=True)
    return exe


def compile_command(gcc, exe, libdir):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return [gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
            "-I", os.path.join(ROOT, "include"), SRC, "-o", exe, "-L", libdir, "-l:libsp24.so",
            f"-Wl,-rpath,{libdir}", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
            f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]


@pytest.mark.parametrize("R,C,T", [(64, 64, 128), (256, 512, 300), (1024, 768, 517), (96, 160, 0)])
def test_plain_c_client_runs_the_hot_path(tmp_path, R, C, T):
    exe = client(tmp_path)
    seed = R * 7 + C + T
    W = WL.normal_f16(seed, 1, (R, C), 0.02)
    X = WL.normal_f16(seed, 3, (T, C))
    dY = WL.normal_f16(seed, 5, (T, R))
    for name, a in (("W", W), ("X", X), ("dY", dY)):
        np.ascontiguousarray(a).tofile(str(tmp_path / f"{name}.bin"))
    print(f"hot_path R={R} C={C} T={T}", flush=True)
    run = subprocess.run([exe, str(tmp_path), str(R), str(C), str(T)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr

    def read(name, dtype, shape):
        return np.fromfile(str(tmp_path / f"{name}.bin"), dtype=dtype).reshape(shape)

    idx = O.mask_search(W)
    assert (read("idx", np.uint8, idx.shape) == idx).all()
    want = O.compress(W, idx)
    for k, dtype in (("vals_row", np.uint16), ("meta_row", np.uint16), ("vals_col", np.uint16),
                     ("meta_col", np.uint16)):
        got = from_blocked(read(k, dtype, want[k].shape), block_width(k))
        assert (got == want[k].view(np.uint16)).all(), k
    if T == 0:
        return
    Y = read("Y", np.float16, (T, R))
    dX = read("dX", np.float16, (T, C))
    for out, ref in ((Y, O.spmm_fwd(X, want["vals_row"], want["meta_row"], R, C)),
                     (dX, O.spmm_bwd_input(dY, want["vals_col"], want["meta_col"], R, C))):
        mr, ma = O.gemm_errors(out.astype(np.float64), ref)
        assert mr <= MAX_REL and ma <= MEAN_ABS, (mr, ma)
