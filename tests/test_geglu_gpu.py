"""GPU parity of the GEGLU forward and backward kernels.

The oracle computes in float64 with the exact GELU; the kernels compute in
fp32 (a fitted erfc and the hardware exponential, within 7e-7 relative over
every fp16 gate) and round the result to fp16.  So each output
must lie within half an fp16 ulp of the exact value, plus the fp32 error of
the few operations before that rounding, plus 2^-25 absolute (below the
smallest fp16 subnormal step).  The fp32 error is 2e-6 relative for
GELU(gate) and the value gradient.  The gate gradient
dout * value * (Phi(x) + x phi(x)) is different: its bracket has a root near
x = -0.75, where the two terms cancel.  Its fp32 error is therefore bounded
in absolute terms, 1e-6 * |dout * value| * (Phi(x) + |x| phi(x)) (about 16
fp32 ulps of the larger term).  Inputs are seeded draws, with
large-magnitude and signed-zero entries mixed in.  Results must not depend on
the layout group.
"""
import math

import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

from gpu_checks import Guarded

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sp():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd import sp24
    sp24.lib()
    return sp24


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def ulp16(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -24)))
    return np.where(a >= 2.0 ** -14, 2.0 ** (e - 10), 2.0 ** -24)


def check(got, want, extra=0.0):
    got = got.astype(np.float64)
    bound = 0.5 * ulp16(want) + 2e-6 * np.abs(want) + 2.0 ** -25 + extra
    # round to nearest even takes fp16 magnitudes from 65520 up to infinity
    overflow_ok = np.isinf(got) & (np.sign(got) == np.sign(want)) & (np.abs(want) >= 65520.0 - bound)
    bad = np.argwhere((np.abs(got - want) > bound) & ~overflow_ok)
    assert bad.size == 0, f"{len(bad)} outside, first {bad[:3].tolist()}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


def gate_grad_slack(U, d, group):
    """Absolute fp32 error budget of each entry of dU (zero on value columns)."""
    T, two_h = U.shape
    blocks = U.astype(np.float64).reshape(T, two_h // (2 * group), 2, group)
    v, x = blocks[:, :, 0, :].reshape(T, -1), blocks[:, :, 1, :].reshape(T, -1)
    cdf = 0.5 * np.vectorize(math.erfc)(-x / math.sqrt(2.0))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    slack = 1e-6 * np.abs(d.astype(np.float64) * v) * (cdf + np.abs(x) * pdf)
    out = np.zeros((T, two_h // (2 * group), 2, group))
    out[:, :, 1, :] = slack.reshape(T, -1, group)
    return out.reshape(T, two_h)


def draw(seed, T, h):
    U = WL.normal_f16(seed, 1, (T, 2 * h))
    d = WL.normal_f16(seed, 2, (T, h))
    rng = np.random.default_rng(seed)
    # edge values: zeros of both signs, large magnitudes, tiny ones
    edges = np.array([0.0, -0.0, 6.0, -6.0, 12.5, -12.5, 40.0, -40.0, 2.0 ** -20, -(2.0 ** -20), 3.0, -3.0],
                     dtype=np.float16)
    m = rng.random(U.shape) < 0.05
    U[m] = rng.choice(edges, size=int(m.sum()))
    return U, d


# Groups of 8, 16 and 32 columns stage a whole wave's backward outputs in LDS
# (64 vectors of 8 units); (40, 256, 8) and (9, 800, 32) have whole waves, and
# the latter a partial last wave as well, like (33, 6400, 16).
@pytest.mark.parametrize("T,h,group", [(1, 8, 8), (3, 64, 16), (7, 48, 48), (5, 96, 32), (64, 512, 16),
                                       (40, 256, 8), (9, 800, 32), (11, 960, 40), (33, 6400, 16), (17, 6400, 6400)])
def test_geglu_forward_backward(sp, T, h, group):
    U, d = draw(T * 131 + h + group, T, h)
    g_out, g_dU = Guarded((T, h), torch.float16), Guarded((T, 2 * h), torch.float16)
    sp.sp24_geglu_fwd(dev(U), group, out=g_out.t)
    sp.sp24_geglu_bwd(dev(U), dev(d), group, dU=g_dU.t)
    g_out.check("out")
    g_dU.check("dU")
    check(g_out.t.cpu().numpy(), O.geglu_fwd(U, group))
    check(g_dU.t.cpu().numpy(), O.geglu_bwd(U, d, group), gate_grad_slack(U, d, group))


@pytest.mark.parametrize("value,limit", [(1.0, None), (-0.75, None), (3000.0, 16.0)])
def test_geglu_every_fp16_gate(sp, value, limit):
    """Every finite fp16 gate (within |gate| <= limit, so value * GELU(gate)
    stays finite), 16 per token, with one value throughout: the GELU
    evaluation checked exhaustively over its fp16 domain, forward and
    backward."""
    g = np.arange(65536, dtype=np.uint16).view(np.float16)
    g = g[np.isfinite(g)]
    if limit is not None:
        g = g[np.abs(g.astype(np.float32)) <= limit]
    g = np.concatenate([g, np.zeros((-len(g)) % 16, np.float16)])
    T = len(g) // 16
    U = np.empty((T, 32), np.float16)
    U[:, :16] = np.float16(value)
    U[:, 16:] = g.reshape(T, 16)
    d = WL.normal_f16(91, 1, (T, 16))
    out = sp.sp24_geglu_fwd(dev(U), 16).cpu().numpy()
    check(out, O.geglu_fwd(U, 16))
    dU = sp.sp24_geglu_bwd(dev(U), dev(d), 16).cpu().numpy()
    check(dU, O.geglu_bwd(U, d, 16), gate_grad_slack(U, d, 16))


def test_geglu_infinite_gates(sp):
    """Gates of +-inf (an fp16 overflow upstream) give what x * Phi(x) gives in
    IEEE arithmetic: GELU(+inf) = +inf, GELU(-inf) = -inf * 0 = NaN; and the
    gate gradient Phi + x phi is NaN at both (inf * 0)."""
    T, h = 4, 16
    U = WL.normal_f16(92, 1, (T, 2 * h))
    U[:, h:] = np.float16(0.5)
    U[0, h:h + 4] = np.float16(np.inf)
    U[1, h:h + 4] = np.float16(-np.inf)
    U[2, h] = np.float16(64.0)
    U[2, h + 1] = np.float16(-64.0)
    d = WL.normal_f16(92, 2, (T, h))
    with np.errstate(invalid="ignore", over="ignore"):
        want_out = O.geglu_fwd(U, h)
        want_dU = O.geglu_bwd(U, d, h)
    got_out = sp.sp24_geglu_fwd(dev(U), h).cpu().numpy().astype(np.float64)
    got_dU = sp.sp24_geglu_bwd(dev(U), dev(d), h).cpu().numpy().astype(np.float64)
    for got, want in ((got_out, want_out), (got_dU, want_dU)):
        assert (np.isnan(got) == np.isnan(want)).all()
        fin = np.isfinite(want)
        assert (got[~fin & ~np.isnan(want)] == want[~fin & ~np.isnan(want)]).all()
        check(got[fin], want[fin])


def test_geglu_layout_group_does_not_change_results(sp):
    T, h = 40, 256
    U, d = draw(3, T, h)
    v, g = U[:, :h], U[:, h:]
    # the same values laid out in blocks of 16
    U16 = np.concatenate([np.concatenate([v[:, 16 * b: 16 * b + 16], g[:, 16 * b: 16 * b + 16]], axis=1)
                          for b in range(h // 16)], axis=1)
    a = sp.sp24_geglu_fwd(dev(U), h)
    b = sp.sp24_geglu_fwd(dev(U16), 16)
    assert torch.equal(a, b)
    da = sp.sp24_geglu_bwd(dev(U), dev(d), h).cpu().numpy()
    db = sp.sp24_geglu_bwd(dev(U16), dev(d), 16).cpu().numpy()
    db_halves = np.concatenate([db.reshape(T, h // 16, 2, 16)[:, :, 0, :].reshape(T, h),
                                db.reshape(T, h // 16, 2, 16)[:, :, 1, :].reshape(T, h)], axis=1)
    assert (da.view(np.uint16) == db_halves.view(np.uint16)).all()


def test_geglu_empty(sp):
    U = torch.empty(0, 32, dtype=torch.float16, device="cuda")
    assert sp.sp24_geglu_fwd(U, 16).shape == (0, 16)
    assert sp.sp24_geglu_bwd(U, torch.empty(0, 16, dtype=torch.float16, device="cuda"), 16).shape == (0, 32)


@pytest.mark.parametrize("group", [16, 6400])
def test_geglu_full_size_sampled(sp, group):
    """A GPT-2-1.5B-wide GEGLU (h = 6400) over 16384 tokens; guard bands around
    both outputs, 64 sampled token rows checked against the oracle."""
    T, h = 16384, 6400
    U = WL.normal_f16(70, 1, (T, 2 * h))
    d = WL.normal_f16(70, 2, (T, h))
    g_out, g_dU = Guarded((T, h), torch.float16), Guarded((T, 2 * h), torch.float16)
    out = sp.sp24_geglu_fwd(dev(U), group, out=g_out.t)
    dU = sp.sp24_geglu_bwd(dev(U), dev(d), group, dU=g_dU.t)
    g_out.check("out")
    g_dU.check("dU")
    rows = np.sort(np.random.default_rng(group).choice(T, size=64, replace=False))
    ri = torch.from_numpy(rows).cuda()
    check(out[ri].cpu().numpy(), O.geglu_fwd(U[rows], group))
    check(dU[ri].cpu().numpy(), O.geglu_bwd(U[rows], d[rows], group), gate_grad_slack(U[rows], d[rows], group))


# ----------------------------------------------------------------------------
# GEGLU fused into the forward sparse GEMM (W's rows in blocks of 16 values
# then their 16 gates, so U has the group-16 layout).  The fused epilogue
# rounds the products to fp16 and then evaluates the same inlined GELU code
# (erfc_parts and geglu_f16, built without fp contraction) as the GEGLU
# kernel, so its outputs must equal GEMM-then-GEGLU bit for bit.

def _fused_case(sp, T, R, C, seed):
    W = WL.normal_f16(seed, 1, (R, C), 0.02)
    X = WL.normal_f16(seed, 2, (T, C))
    f = sp.sp24_search_compress(dev(W))
    return W, X, f


@pytest.mark.parametrize("T,R,C", [(1, 32, 64), (100, 96, 128), (300, 544, 320), (257, 256, 1024)])
def test_fused_geglu_matches_gemm_then_geglu_bit_for_bit(sp, T, R, C):
    W, X, f = _fused_case(sp, T, R, C, T + R)
    out, U = sp.sp24_spmm_fwd_geglu(dev(X), f["vals_row"], f["meta_row"], R, C, U=True)
    Y = sp.sp24_spmm_fwd(dev(X), f["vals_row"], f["meta_row"], R, C)
    assert torch.equal(U, Y)
    assert torch.equal(out, sp.sp24_geglu_fwd(Y, 16))
    check(out.cpu().numpy(), O.geglu_fwd(U.cpu().numpy(), 16))
    out2, none = sp.sp24_spmm_fwd_geglu(dev(X), f["vals_row"], f["meta_row"], R, C)
    assert none is None and torch.equal(out2, out)
    # against the oracle: GEGLU of the float64 product, to the GEMM tolerance
    c = O.compress(W, O.mask_search(W))
    want = O.geglu_fwd(O.spmm_fwd(X, c["vals_row"], c["meta_row"], R, C), 16)
    mr, ma = O.gemm_errors(out.cpu().numpy().astype(np.float64), want)
    assert mr <= 1e-2 and ma <= 1e-3, (mr, ma)


def test_fused_geglu_fallback_needs_products(sp):
    """K (= C) not a multiple of 64: the library stores U and runs the GEGLU
    kernel on it; without a U buffer it reports UNSUPPORTED."""
    T, R, C = 40, 64, 80
    W, X, f = _fused_case(sp, T, R, C, 5)
    out, U = sp.sp24_spmm_fwd_geglu(dev(X), f["vals_row"], f["meta_row"], R, C, U=True)
    assert torch.equal(out, sp.sp24_geglu_fwd(U, 16))       # this path runs the GEGLU kernel itself
    with pytest.raises(sp.Sp24Error) as e:
        sp.sp24_spmm_fwd_geglu(dev(X), f["vals_row"], f["meta_row"], R, C)
    assert e.value.status == 5


def test_fused_geglu_gpt2_1p5b_shape(sp):
    """W1's shape of the 1.5B FFN (6400 x 1600, read as a gated layer with
    h = 3200) over 16384 tokens: the 256-feature tail split is taken.  Same
    products and the same outputs as the two-kernel path everywhere, nothing
    written outside U or out (guard bands), the oracle on sampled rows."""
    cfg = WL.GPT2_1P5B
    inp = WL.ffn_inputs(cfg)
    R, C = inp.w1.shape
    T = inp.x.shape[0]
    f = sp.sp24_search_compress(dev(inp.w1))
    dX = dev(inp.x)
    gout, gU = Guarded((T, R // 2), torch.float16), Guarded((T, R), torch.float16)
    out, U = sp.sp24_spmm_fwd_geglu(dX, f["vals_row"], f["meta_row"], R, C, out=gout.t, U=gU.t)
    gout.check("out")
    gU.check("U")
    Y = sp.sp24_spmm_fwd(dX, f["vals_row"], f["meta_row"], R, C)
    assert torch.equal(U, Y)
    assert torch.equal(out, sp.sp24_geglu_fwd(Y, 16))
    # without U: the same outputs, and still nothing outside out
    gout2 = Guarded((T, R // 2), torch.float16)
    sp.sp24_spmm_fwd_geglu(dX, f["vals_row"], f["meta_row"], R, C, out=gout2.t)
    gout2.check("out (no U)")
    assert torch.equal(gout2.t, out)
    rows = np.sort(np.random.default_rng(4).choice(inp.x.shape[0], size=32, replace=False))
    c = O.compress(inp.w1, O.mask_search(inp.w1))
    want = O.geglu_fwd(O.spmm_fwd(inp.x[rows], c["vals_row"], c["meta_row"], R, C), 16)
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    mr, ma = O.gemm_errors(got, want)
    assert mr <= 1e-2 and ma <= 1e-3, (mr, ma)
