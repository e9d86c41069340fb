"""One training step of a gated 2:4-sparse FFN layer, composed from the
library's entry points (sp24.py; every step runs in the HIP kernels).

"Accelerating Transformer Pre-training with 2:4 Sparsity" trains the FFN
linears with transposable 2:4 masks recomputed from the dense weights every
step, uses the column form of the same mask for the input gradient, adds the
masked decay term to the weight gradient, and accelerates the gated
activation (abstract; the reproducibility table's "Software Dependencies"
row).  The layer here is

    U  = X W1s^T              [T, 2h]  (W1's rows: blocks of 16 value rows, then the 16 gate rows)
    Hg = value * GELU(gate)   [T, h]   (fused into the first GEMM's epilogue)
    Y  = Hg W2s^T             [T, d]

and its backward

    dHg = dY W2s,   dW2 = dY^T Hg + decay (1 - M2) W2
    dU  = GEGLU'(U, dHg)
    dX  = dU W1s,   dW1 = dU^T X  + decay (1 - M1) W1

with W1 [2h, d] and W2 [d, h] the dense fp16 master weights, Ms their masks.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import sp24

GROUP = 16


@dataclass
class Saved:
    X: torch.Tensor
    U: torch.Tensor
    Hg: torch.Tensor


class SparseGegluFFN:
    """W1 fp16 [2h, d] in blocks of 16 value rows then 16 gate rows, W2 fp16
    [d, h]; h a multiple of 16.  `refresh()` searches and compresses both
    weights (and adds each weight's flipped mask entries to `flips` once
    masks exist); `forward` and `backward` run the step."""

    def __init__(self, W1: torch.Tensor, W2: torch.Tensor, decay: float = 0.0):
        two_h, d = W1.shape
        if W2.shape != (d, two_h // 2) or two_h % 32 != 0:
            raise ValueError("W1 must be [2h, d] with 2h a multiple of 32, W2 [d, h]")
        self.W1, self.W2, self.decay = W1, W2, float(decay)
        self.forms = None
        self.flips = torch.zeros(2, dtype=torch.int64, device=W1.device)
        self._side = None

    def refresh(self) -> None:
        if self.forms is None:
            self.forms = sp24.sp24_search_compress_batch([self.W1, self.W2])
        else:
            self.forms = sp24.sp24_search_compress_batch(
                [self.W1, self.W2], outs=self.forms, prev=[f["idx"] for f in self.forms],
                flips=[self.flips[0:1], self.flips[1:2]])

    def _current_forms(self):
        if self.forms is None:
            raise RuntimeError("call refresh() first: the layer has no compressed weights yet")
        return self.forms

    def forward(self, X: torch.Tensor):
        f1, f2 = self._current_forms()
        two_h, d = self.W1.shape
        Hg, U = sp24.sp24_spmm_fwd_geglu(X, f1["vals_row"], f1["meta_row"], two_h, d, U=True)
        Y = sp24.sp24_spmm_fwd(Hg, f2["vals_row"], f2["meta_row"], d, two_h // 2)
        return Y, Saved(X, U, Hg)

    def backward(self, dY: torch.Tensor, saved: Saved):
        """dW2 runs on a second stream beside dHg, the GEGLU backward and dX,
        which do not need it: its last round of tiles leaves most CUs to
        them.  The caller's stream waits for it before this returns, and
        every output is allocated on the caller's stream."""
        f1, f2 = self._current_forms()
        two_h, d = self.W1.shape
        main = torch.cuda.current_stream()
        if self._side is None:
            self._side = torch.cuda.Stream(device=main.device)
        side = self._side
        dW2 = torch.empty(d, two_h // 2, dtype=torch.float32, device=dY.device)
        dHg = sp24.sp24_spmm_bwd_input(dY, f2["vals_col"], f2["meta_col"], d, two_h // 2)
        side.wait_stream(main)
        sp24.sp24_weight_grad(dY, saved.Hg, self.W2, f2["idx"], self.decay, dW=dW2, stream=side)
        dU = sp24.sp24_geglu_bwd(saved.U, dHg, GROUP)
        dX = sp24.sp24_spmm_bwd_input(dU, f1["vals_col"], f1["meta_col"], two_h, d)
        dW1 = sp24.sp24_weight_grad(dU, saved.X, self.W1, f1["idx"], self.decay)
        main.wait_stream(side)
        return dX, dW1, dW2
