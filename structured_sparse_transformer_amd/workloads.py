"""Seeded synthetic workloads for the transposable 2:4 FFN path.

This module only draws inputs. It holds none of the method's arithmetic, so
both the CPU oracle's tests and the HIP path's tests and benchmark can use it.

The paper ("Accelerating Transformer Pre-training with 2:4 Sparsity",
reproducibility table, "Open Datasets" and "Hardware Specification" rows)
trains GPT-2 124M/355M/774M/1.5B on OpenWebText. Neither the dataset nor
trained weights are available here, so every input is a seeded draw with the
shapes of one GPT-2 FFN layer:

* weights ``W1 [4d, d]`` and ``W2 [d, 4d]`` (PyTorch ``Linear`` layout
  ``[out, in]``), fp16 ``N(0, 0.02)`` (GPT-2's init scale);
* activations ``X [T, d]`` and ``H [T, 4d]`` and output gradients
  ``dY1 [T, 4d]``, ``dY2 [T, d]``, fp16 ``N(0, 1)``; ``T = 16384`` tokens.

Draw recipe: ``numpy.random.default_rng([base, k])``, ``standard_normal`` in
float32, times sigma, rounded to fp16 (round to nearest even).  ``base`` is the
configuration's seed; ``k`` names the tensor (1 W1, 2 W2, 3 X, 4 H, 5 dY1,
6 dY2, 100+s the step-s weight noise).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

K_W1, K_W2, K_X, K_H, K_DY1, K_DY2, K_NOISE0 = 1, 2, 3, 4, 5, 6, 100
W_SIGMA = 0.02
NOISE_SIGMA = 1e-3


def normal_f16(base: int, k: int, shape, sigma: float = 1.0) -> np.ndarray:
    """fp16 draw of N(0, sigma^2): float32 normal times sigma, then RNE to fp16."""
    rng = np.random.default_rng([base, k])
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return x.astype(np.float16)


def noise_f32(base: int, step: int, shape, sigma: float = NOISE_SIGMA) -> np.ndarray:
    """float32 N(0, sigma^2) weight noise for step ``step`` of the noisy loop."""
    rng = np.random.default_rng([base, K_NOISE0 + step])
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def add_noise_f16(w: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """The stand-in weight update: fp16(f32(w) + noise), round to nearest even."""
    return (w.astype(np.float32) + noise).astype(np.float16)


def random_idx(base: int, k: int, shape, hi: int = 90) -> np.ndarray:
    """Uniform uint8 pattern indices in [0, hi): stand-in mask arrays."""
    rng = np.random.default_rng([base, k])
    return rng.integers(0, hi, size=shape, dtype=np.uint8)


def uniform_f32(base: int, k: int, shape) -> np.ndarray:
    """fp32 uniforms in [0, 1) (the random draws of a stochastic estimator)."""
    rng = np.random.default_rng([base, k])
    return rng.random(shape, dtype=np.float32)


def stress_weight(base: int, R: int = 4096, C: int = 4096) -> np.ndarray:
    """Tie-heavy stress weight.

    Rows [0, R/2): uniform integers in {-3..3} divided by 8 (many equal
    magnitudes, so many tied pattern scores).  Rows [R/2, R): fp16 N(0, 0.02).
    Rows [R/2 - 2, R/2 + 62): every entry exactly 0.0625.  The band is 64 rows
    tall, starts two rows before the seam and so is not 4-row aligned.
    """
    rng = np.random.default_rng([base, K_W1])
    w = np.empty((R, C), dtype=np.float16)
    h = R // 2
    w[:h] = (rng.integers(-3, 4, size=(h, C)).astype(np.float32) / 8).astype(np.float16)
    w[h:] = normal_f16(base, K_W2, (R - h, C), W_SIGMA)
    lo, hi = max(h - 2, 0), min(h + 62, R)
    w[lo:hi] = np.float16(0.0625)
    return w


@dataclass(frozen=True)
class FFNConfig:
    """One GPT-2-shaped FFN layer workload."""
    name: str
    seed: int
    d: int            # model width; the FFN is d -> 4d -> d
    tokens: int
    steps: int = 1    # noisy re-search steps (the 1.5B loop uses 20)
    hidden: int = 0   # 4d unless given

    @property
    def dff(self) -> int:
        return self.hidden or 4 * self.d

    def gemm_shapes(self):
        """(name, T, N_out, K) of the four sparse GEMMs of one step."""
        T, d, f = self.tokens, self.d, self.dff
        return [("fwd1", T, f, d), ("bwd1", T, d, f), ("fwd2", T, d, f), ("bwd2", T, f, d)]

    def dense_equiv_flops(self) -> int:
        return sum(2 * T * N * K for _, T, N, K in self.gemm_shapes())


TINY = FFNConfig("tiny", 1001, 64, 128, hidden=64)
GPT2_355M = FFNConfig("gpt2-355m-ffn", 1003, 1024, 16384)
GPT2_774M = FFNConfig("gpt2-774m-ffn", 1004, 1280, 16384)
GPT2_1P5B = FFNConfig("gpt2-1.5b-ffn", 1005, 1600, 16384, steps=20)
STRESS_SEED = 1002
CONFIGS = {c.name: c for c in (TINY, GPT2_355M, GPT2_774M, GPT2_1P5B)}


@dataclass
class FFNInputs:
    w1: np.ndarray
    w2: np.ndarray
    x: np.ndarray
    h: np.ndarray
    dy1: np.ndarray
    dy2: np.ndarray
    extra: dict = field(default_factory=dict)


def ffn_weights(cfg: FFNConfig):
    d, f = cfg.d, cfg.dff
    return (normal_f16(cfg.seed, K_W1, (f, d), W_SIGMA),
            normal_f16(cfg.seed, K_W2, (d, f), W_SIGMA))


def ffn_inputs(cfg: FFNConfig, tokens: int | None = None) -> FFNInputs:
    """All tensors of one FFN-layer step. ``tokens`` truncates T (row prefix)."""
    T = cfg.tokens if tokens is None else tokens
    d, f = cfg.d, cfg.dff
    w1, w2 = ffn_weights(cfg)
    full = cfg.tokens
    x = normal_f16(cfg.seed, K_X, (full, d))[:T]
    h = normal_f16(cfg.seed, K_H, (full, f))[:T]
    dy1 = normal_f16(cfg.seed, K_DY1, (full, f))[:T]
    dy2 = normal_f16(cfg.seed, K_DY2, (full, d))[:T]
    return FFNInputs(w1, w2, np.ascontiguousarray(x), np.ascontiguousarray(h),
                     np.ascontiguousarray(dy1), np.ascontiguousarray(dy2))


def noisy_weights(cfg: FFNConfig, w: np.ndarray, which: int, steps: int):
    """Weights of the noisy loop: step s uses fp16(f32(W_{s-1}) + noise_s).

    ``which`` (1 or 2) keeps the two weights' noise streams apart.
    Yields (step, weight) for step = 0 .. steps-1.
    """
    cur = w
    for s in range(steps):
        n = noise_f32(cfg.seed * 10 + which, s, w.shape)
        cur = add_noise_f16(cur, n)
        yield s, cur
