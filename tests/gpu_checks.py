"""Whole-output comparisons and guard bands shared by the GPU parity tests.

``gemm_full`` compares every element of a device GEMM output with the
oracle's float64 product, a chunk of token rows at a time so that host memory
stays bounded; the errors are accumulated over the whole output, so the
normwise maximum relative error and the mean absolute error are those of the
full matrices, exactly as ``oracle.gemm_errors`` defines them.

``Guarded`` allocates an output inside a larger device buffer whose bytes
before and after it hold a sentinel, so that a test can check that a kernel
wrote nothing outside the output it was given.  The guard is 4 KiB on each
side, which keeps the output's 16-byte (indeed 4 KiB) alignment.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import sp24_oracle as O

MAX_REL, MEAN_ABS = 1e-2, 1e-3
GUARD = 4096
SENTINEL = 0xA5


def host_rows(out_dev, lo: int, hi: int) -> np.ndarray:
    return out_dev[lo:hi].float().cpu().numpy().astype(np.float64)


def gemm_full(out_dev, A: np.ndarray, vals, meta, R: int, C: int, fwd: bool, chunk: int = 4096,
              max_rel: float = MAX_REL, mean_abs: float = MEAN_ABS):
    """Every element of ``out_dev`` ([T, N] fp16 on the GPU) against the oracle:
    ``A Ws^T`` from the row form when ``fwd``, ``A Ws`` from the column form
    otherwise.  Returns (normwise max relative error, mean absolute error)."""
    T = A.shape[0]
    assert out_dev.shape[0] == T
    f = O.spmm_fwd if fwd else O.spmm_bwd_input
    max_diff = max_ref = sum_diff = 0.0
    n = 0
    for lo in range(0, T, chunk):
        hi = min(T, lo + chunk)
        ref = f(A[lo:hi], vals, meta, R, C)
        got = host_rows(out_dev, lo, hi)
        assert got.shape == ref.shape
        d = np.abs(got - ref)
        max_diff = max(max_diff, float(d.max()))
        max_ref = max(max_ref, float(np.abs(ref).max()))
        sum_diff += float(d.sum())
        n += d.size
    mr = max_diff / max_ref if max_ref > 0 else max_diff
    ma = sum_diff / n if n else 0.0
    assert mr <= max_rel and ma <= mean_abs, (mr, ma)
    return mr, ma


class Guarded:
    """A device output of ``shape`` and ``dtype`` with sentinel bytes around it.

    ``fill`` (a byte) is written into the output region as well, so a test can
    also tell an element the kernel never wrote."""

    def __init__(self, shape, dtype, fill: int = SENTINEL, device: str = "cuda"):
        self.shape = tuple(int(s) for s in shape)
        self.dtype = dtype
        self.nbytes = int(np.prod(self.shape)) * torch.empty(0, dtype=dtype).element_size()
        self.raw = torch.full((self.nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=device)
        if fill != SENTINEL:
            self.raw[GUARD:GUARD + self.nbytes].fill_(fill)
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(self.shape)

    def check(self, name: str = "output") -> None:
        """Both guard bands still hold the sentinel."""
        torch.cuda.synchronize()
        lo = self.raw[:GUARD].cpu().numpy()
        hi = self.raw[GUARD + self.nbytes:].cpu().numpy()
        bad_lo = np.flatnonzero(lo != SENTINEL)
        bad_hi = np.flatnonzero(hi != SENTINEL)
        assert bad_lo.size == 0, f"{name}: {bad_lo.size} bytes written before the output (last at -{GUARD - bad_lo[-1]})"
        assert bad_hi.size == 0, f"{name}: {bad_hi.size} bytes written after the output (first at +{bad_hi[0]})"


def guarded_forms(R: int, C: int, idx: bool = True) -> dict:
    """Guarded outputs of a search + compression of an [R, C] weight."""
    spec = {"vals_row": ((R, C // 2), torch.float16), "meta_row": ((R, C // 16), torch.int16),
            "vals_col": ((C, R // 2), torch.float16), "meta_col": ((C, R // 16), torch.int16)}
    if idx:
        spec["idx"] = ((R // 4, C // 4), torch.uint8)
    return {k: Guarded(shape, dt) for k, (shape, dt) in spec.items()}


def check_all(guards: dict) -> None:
    for k, g in guards.items():
        g.check(k)
