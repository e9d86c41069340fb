"""Host model of the kernels' GELU evaluation (gelu_cdf / gelu_cdf_pdf in
sp24_device.hpp): the fitted erfc polynomial and the fp32 operation sequence,
emulated in numpy over every finite fp16 input.

numpy float32 rounds each operation; an FMA is one float64 product-sum
rounded once to fp32, and the hardware 2^y is the correctly rounded value
scaled by 1 +- 2 ulp, to cover its documented error.  The reference is
scipy's float64 erfc.  This checks the design's accuracy claims (the fit
within 1.2e-7, Phi within 7e-7, phi within 7.5e-7 relative) on the CPU; the
GPU test test_geglu_every_fp16_gate checks the kernels themselves.
"""
import pathlib
import re

import numpy as np
import pytest

scipy_special = pytest.importorskip("scipy.special")

HEADER = pathlib.Path(__file__).resolve().parents[1] / "structured_sparse_transformer_amd" / "csrc" / "sp24_device.hpp"
f32 = np.float32


def header_constants():
    text = HEADER.read_text()
    body = re.search(r"kErfcP\[10\]\s*=\s*\{([^}]*)\}", text).group(1)
    coef = [f32(float(v.strip().rstrip("f"))) for v in body.split(",")]
    named = {}
    for name in ("kLog2E", "kLog2ELo", "kLn2", "kInvSqrt2", "kInvSqrt2Pi"):
        named[name] = f32(float(re.search(name + r"\s*=\s*([-0-9.e]+)f", text).group(1)))
    assert len(coef) == 10
    return coef, named


def fma(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(f32)


def exp2_hw(y, ulps):
    with np.errstate(under="ignore", over="ignore"):
        return (np.exp2(np.asarray(y, np.float64)) * (1.0 + ulps * 2.0 ** -23)).astype(f32)


def model(x, ulps):
    coef, k = header_constants()
    xs = x
    x = np.clip(x, f32(-64), f32(64)).astype(f32)      # the kernel clamps the erfc argument
    z = (np.abs(x) * k["kInvSqrt2"]).astype(f32)
    t = (1.0 / fma(f32(0.5), z, f32(1)).astype(np.float64)).astype(f32)
    p = np.full_like(t, coef[9])
    for c in coef[8:0:-1]:
        p = fma(p, t, c)
    p = fma(p, t, f32(coef[0] - k["kLn2"]))      # the halving folded into the constant term
    hi = (x * x).astype(f32)
    lo = fma(x, x, -hi)
    a = (f32(-0.5) * hi).astype(f32)
    s = (a + p).astype(f32)
    e = fma(f32(-0.5), lo, (p - (s - a).astype(f32)).astype(f32))
    yh = (s * k["kLog2E"]).astype(f32)
    yl = fma(s, k["kLog2ELo"], fma(s, k["kLog2E"], -yh))
    E = exp2_hw(yh, ulps)
    ex = fma(E, fma(yl, k["kLn2"], e), E)
    half = (t * ex).astype(f32)
    cdf = np.where(xs < 0, half, (f32(1) - half).astype(f32))
    pdf = ((ex * exp2_hw((-p * k["kLog2E"]).astype(f32), ulps)).astype(f32) * k["kInvSqrt2Pi"]).astype(f32)
    return cdf, pdf


def every_fp16():
    x = np.arange(65536, dtype=np.uint16).view(np.float16)
    return x[np.isfinite(x)].astype(f32)


def test_fit_error_of_header_coefficients():
    coef, _ = header_constants()
    t = np.linspace(0.0, 1.0, 100001)
    z = 2.0 * (1.0 - t[1:]) / t[1:]
    target = np.concatenate([[np.log(1.0 / (2.0 * np.sqrt(np.pi)))],
                             np.log(scipy_special.erfcx(z) / t[1:])])
    approx = np.polynomial.polynomial.polyval(t, np.array(coef, np.float64))
    assert np.abs(approx - target).max() < 1.3e-7


@pytest.mark.parametrize("ulps", [0.0, 2.0, -2.0])
def test_cdf_and_pdf_over_every_fp16(ulps):
    x = every_fp16()
    cdf, pdf = model(x, ulps)
    xd = x.astype(np.float64)
    want_cdf = 0.5 * scipy_special.erfc(-xd / np.sqrt(2.0))
    want_pdf = np.exp(-0.5 * xd * xd) / np.sqrt(2.0 * np.pi)
    # relative error wherever the exact value is a normal fp32 number
    for got, want, bound in ((cdf, want_cdf, 7e-7), (pdf, want_pdf, 7.5e-7)):
        ok = want > 1e-37
        rel = np.abs(got[ok].astype(np.float64) - want[ok]) / want[ok]
        assert rel.max() < bound, (rel.max(), x[ok][np.argmax(rel)])
        # beyond that, the result has underflowed to (nearly) zero
        assert np.all(got[~ok] < 1e-37)
