"""Builds libsp24.so (the HIP kernels and their C ABI) in-tree for gfx950.

Run ``python -m structured_sparse_transformer_amd.build``.  hipcc cross-compiles
for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsp24.so")
SOURCES = ["sp24_api.hip", "sp24_search.hip", "sp24_spmm.hip", "sp24_dw.hip", "sp24_act.hip", "sp24_mvue.hip"]
ARCH = os.environ.get("SP24_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++20", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # no fused multiply-add contraction: the mask scores are plain fp32 sums
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
