"""GPU parity of the weight gradient with the masked decay term.

dW = dY^T X + decay * (1 - M) * W against the oracle's float64 value.  The
products of fp16 inputs are exact in fp32 and the GPU sums T of them in fp32
(MFMA blocks of 16, then one accumulator per output): the rounding-error
model of such a sum, sqrt(T / 16 + 4) * 2^-24 * sum|dY x| relative to max|dW|,
is below 1e-5 for the shapes here, so the tests allow a normwise max relative
error of 1e-4 (a dropped token, sign or operand shows up far above it) and a
mean absolute error of 1e-5 of the mean magnitude.  The decay term alone
(T = 0) must match to one fp32 rounding.  Full-size outputs are checked in
full against the oracle, inside guard bands, plus a column-sum identity.
With the two-way token split the two halves' fp32 sums are added once more;
the error model above covers that rounding.
"""
import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

from gpu_checks import Guarded

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
MAX_REL, MEAN_REL = 1e-4, 1e-5


@pytest.fixture(scope="module")
def sp():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd import sp24
    sp24.lib()
    return sp24


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check(got, want):
    got = got.astype(np.float64)
    err = np.abs(got - want)
    max_rel = err.max() / max(np.abs(want).max(), 1e-300)
    mean_rel = err.mean() / max(np.abs(want).mean(), 1e-300)
    assert max_rel <= MAX_REL and mean_rel <= MEAN_REL, (max_rel, mean_rel)


def inputs(seed, T, R, C, wsig=1.0):
    dY = WL.normal_f16(seed, 1, (T, R))
    X = WL.normal_f16(seed, 2, (T, C))
    W = WL.normal_f16(seed, 3, (R, C), wsig)
    return dY, X, W


@pytest.mark.parametrize("T,R,C", [(1, 16, 16), (5, 16, 32), (31, 48, 80), (32, 64, 64), (33, 272, 144),
                                   (100, 528, 336), (257, 160, 256), (700, 256, 160), (64, 1040, 656)])
def test_weight_grad_ragged(sp, T, R, C):
    dY, X, W = inputs(T + R, T, R, C)
    idx = O.mask_search(W)
    decay = 0.75
    g = Guarded((R, C), torch.float32)
    sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), decay, dW=g.t)
    g.check("dW")
    check(g.t.cpu().numpy(), O.weight_grad(dY, X, W, idx, decay))


def test_weight_grad_decay_term_alone(sp):
    """No tokens: dW is the decay term, to one fp32 rounding of decay * w."""
    R, C = 272, 400
    W = WL.normal_f16(5, 3, (R, C), 0.02)
    idx = O.mask_search(W)
    e = torch.empty(0, R, dtype=torch.float16, device="cuda"), torch.empty(0, C, dtype=torch.float16, device="cuda")
    got = sp.sp24_weight_grad(e[0], e[1], dev(W), dev(idx), 1e-3).cpu().numpy().astype(np.float64)
    want = O.weight_grad(np.zeros((0, R), np.float16), np.zeros((0, C), np.float16), W, idx, 1e-3)
    kept = O.idx_to_mask(idx).astype(bool)
    assert (got[kept] == 0).all()
    assert np.allclose(got[~kept], want[~kept], rtol=2 ** -23, atol=0)


def test_weight_grad_no_tokens_no_decay_is_zero(sp):
    e0 = torch.empty(0, 32, dtype=torch.float16, device="cuda")
    e1 = torch.empty(0, 48, dtype=torch.float16, device="cuda")
    out = torch.full((32, 48), 7.0, dtype=torch.float32, device="cuda")
    sp.sp24_weight_grad(e0, e1, dW=out)
    assert (out.cpu().numpy() == 0).all()


def test_weight_grad_large_decay_and_bad_indices(sp):
    """A decay large enough to be seen next to the product, and pattern
    indices >= 90 (read as pattern 0, as the oracle is told here)."""
    T, R, C = 96, 144, 208
    dY, X, W = inputs(8, T, R, C)
    idx = WL.random_idx(8, 4, (R // 4, C // 4), hi=256)
    idx0 = np.where(idx < 90, idx, 0).astype(np.uint8)
    got = sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), 50.0).cpu().numpy()
    check(got, O.weight_grad(dY, X, W, idx0, 50.0))
    plain = sp.sp24_weight_grad(dev(dY), dev(X)).cpu().numpy()
    check(plain, O.weight_grad(dY, X, None, None, 0.0))


def test_weight_grad_deterministic(sp):
    T, R, C = 2048, 512, 384
    dY, X, W = inputs(9, T, R, C)
    idx = O.mask_search(W)
    a = sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), 0.1)
    b = sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), 0.1)
    assert torch.equal(a, b)
    check(a.cpu().numpy(), O.weight_grad(dY, X, W, idx, 0.1))


@pytest.mark.parametrize("T,R,C", [(976, 3072, 2560), (40, 3072, 2560), (976, 2560, 3072)])
def test_weight_grad_token_split(sp, T, R, C):
    """Shapes whose tiles take the two-way token split (96 whole 256 x 320 or
    320 x 256 tiles, 192 workgroups): an odd number of 32-token stages (31:
    the first half gets 15, the second 16) and two stages.  Every element
    against the oracle inside guard bands, and the same bits on a second call
    (the halves meet through a flag; their sum does not depend on which
    finishes first)."""
    dY, X, W = inputs(T + R + C, T, R, C, 0.02)
    idx = O.mask_search(W)
    g = Guarded((R, C), torch.float32)
    sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), 0.05, dW=g.t)
    g.check("dW")
    got = g.t.cpu().numpy()
    check(got, O.weight_grad(dY, X, W, idx, 0.05))
    again = sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), 0.05)
    assert torch.equal(again, g.t)


def test_weight_grad_token_split_on_two_streams(sp):
    """Split launches of two weights in flight together on two streams (they
    take different sets of tile flags), then again in the other order."""
    T, R, C = 976, 3072, 2560
    cases = [inputs(70 + k, T, R, C, 0.02) for k in range(2)]
    idxs = [O.mask_search(W) for _, _, W in cases]
    devs = [(dev(dY), dev(X), dev(W), dev(i)) for (dY, X, W), i in zip(cases, idxs)]
    wants = [O.weight_grad(dY, X, W, i, 0.05) for (dY, X, W), i in zip(cases, idxs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for order in ((0, 1), (1, 0)):
        outs = [torch.empty(R, C, dtype=torch.float32, device="cuda") for _ in range(2)]
        torch.cuda.synchronize()
        for k in order:
            with torch.cuda.stream(streams[k]):
                sp.sp24_weight_grad(*devs[k][:3], devs[k][3], 0.05, dW=outs[k])
        torch.cuda.synchronize()
        for k in range(2):
            check(outs[k].cpu().numpy(), wants[k])


def _column_sums(got, dY, X, W, idx, decay):
    """sum_r dW[r, c] = (sum_r dY[t, r]) . X[:, c] + sum_r decay-term (an extra
    check beside the elementwise one)."""
    dY64, X64 = dY.astype(np.float64), X.astype(np.float64)
    masks = O.idx_to_mask(idx)
    colsum = dY64.sum(axis=1) @ X64 + decay * ((1.0 - masks) * W.astype(np.float64)).sum(axis=0)
    err = np.abs(got.astype(np.float64).sum(axis=0) - colsum).max() / np.abs(colsum).max()
    assert err <= 1e-4, err


@pytest.mark.parametrize("cfg", [WL.GPT2_355M, WL.GPT2_774M, WL.GPT2_1P5B], ids=lambda c: c.name)
def test_weight_grad_ffn_configs(sp, cfg):
    """Both weight gradients of one FFN layer at 16384 tokens: dW1 = dY1^T X
    (shape of W1) and dW2 = dY2^T H (shape of W2), with the decay term; every
    element against the oracle, guard bands around each output."""
    inp = WL.ffn_inputs(cfg)
    decay = 2e-4
    for (dY, A, W) in ((inp.dy1, inp.x, inp.w1), (inp.dy2, inp.h, inp.w2)):
        R, C = W.shape
        print(f"{cfg.name} dW {R}x{C}", flush=True)
        idx = O.mask_search(W)
        g = Guarded((R, C), torch.float32)
        sp.sp24_weight_grad(dev(dY), dev(A), dev(W), dev(idx), decay, dW=g.t)
        g.check("dW")
        got = g.t.cpu().numpy()
        check(got, O.weight_grad(dY, A, W, idx, decay))
        _column_sums(got, dY, A, W, idx, decay)


def test_weight_grad_square_4096(sp):
    """A 4096 x 4096 weight (the 256 x 256 tile shape) at 2048 tokens, checked in full."""
    T, R, C = 2048, 4096, 4096
    dY, X, W = inputs(11, T, R, C, 0.02)
    idx = O.mask_search(W)
    got = sp.sp24_weight_grad(dev(dY), dev(X), dev(W), dev(idx), 0.01).cpu().numpy()
    check(got, O.weight_grad(dY, X, W, idx, 0.01))
