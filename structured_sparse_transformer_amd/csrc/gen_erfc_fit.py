"""Fit of the erfc polynomial used by gelu_cdf (sp24_device.hpp).

erfc(z) = t * exp(-z^2 + P(t)) with t = 1 / (1 + z/2), z >= 0, so P(t) =
log(erfcx(z) / t), where erfcx(z) = exp(z^2) erfc(z) is smooth and z =
2 (1 - t) / t maps t in (0, 1] onto z in [0, inf).  At t = 0 the limit is
log(1 / (2 sqrt(pi))).  The degree-9 polynomial comes from least squares on
Chebyshev nodes, reweighted toward the largest errors (Lawson's iteration)
so that it approaches the minimax fit.  Prints the coefficients (lowest
degree first, as fp32 literals) and the largest error on a fine grid.

Run: python gen_erfc_fit.py   (needs numpy and scipy)
"""
import numpy as np
from scipy.special import erfcx

DEGREE = 9


def target(t):
    t = np.asarray(t, np.float64)
    out = np.full_like(t, np.log(1.0 / (2.0 * np.sqrt(np.pi))))
    pos = t > 1e-12
    z = 2.0 * (1.0 - t[pos]) / t[pos]
    out[pos] = np.log(erfcx(z) / t[pos])
    return out


def fit(degree=DEGREE, nodes=4000, rounds=60):
    x = 0.5 - 0.5 * np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes)
    V = np.vander(x, degree + 1, increasing=True)
    y = target(x)
    w = np.ones(nodes)
    for _ in range(rounds):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(V * sw[:, None], y * sw, rcond=None)
        err = np.abs(V @ c - y)
        w = np.maximum(w * err / err.sum() * nodes, 1e-12)
    return c


if __name__ == "__main__":
    c = fit()
    grid = np.linspace(0.0, 1.0, 200001)
    worst = np.abs(np.polynomial.polynomial.polyval(grid, c.astype(np.float32).astype(np.float64)) - target(grid)).max()
    print(", ".join(np.format_float_positional(np.float32(v), unique=True) + "f" for v in c))
    print(f"largest error of P with fp32 coefficients: {worst:.2e}")
