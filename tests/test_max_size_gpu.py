"""The sparse GEMMs and the weight gradient at the largest sizes their fast
kernels accept, and the GEMM just past that size.

The fast kernels address the token-major operand with 32-bit byte offsets
from its base.  The GEMMs use them while T*K*2 < 2^31 bytes and switch to
the generic kernel, which uses 64-bit indices, above that.  The weight
gradient needs T*R and T*C below 2^30 elements and refuses anything larger.
One 16401 x 65472 fp16 draw (2.1 GB) feeds every case here.  Every output
element is checked against the oracle (over chunks of token rows), inside
guard bands; the last token rows sit at the top of the offset range.
"""
import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

from forms_layout import forms_to_blocked
from gpu_checks import Guarded, gemm_full

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
MAX_REL, MEAN_ABS = 1e-2, 1e-3
DW_MAX_REL = 1e-4
T_FAST, T_GENERIC, K_BIG, N = 16384, 16401, 65472, 256
SEED = 77


@pytest.fixture(scope="module")
def sp():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd import sp24
    sp24.lib()
    return sp24


@pytest.fixture(scope="module")
def big():
    # the fast GEMM takes the first T_FAST rows, the generic one all of them
    assert T_FAST * K_BIG * 2 < 2 ** 31 <= T_GENERIC * K_BIG * 2
    a = WL.normal_f16(SEED, 1, (T_GENERIC, K_BIG))
    return a, torch.from_numpy(a).cuda()


@pytest.fixture(scope="module")
def forms():
    """The oracle's row form of a [256, 65472] weight, on the host and the GPU."""
    W = WL.normal_f16(SEED, 2, (N, K_BIG), 0.02)
    c = O.compress(W, O.mask_search(W))
    b = forms_to_blocked(c)   # the library's order
    return c, (torch.from_numpy(b["vals_row"]).cuda(), torch.from_numpy(b["meta_row"].view(np.int16)).cuda())


@pytest.mark.parametrize("T", [T_FAST, T_GENERIC])
def test_spmm_fwd_at_the_offset_limit(sp, big, forms, T):
    a, a_dev = big
    c, (vals, meta) = forms
    g = Guarded((T, N), torch.float16)
    sp.sp24_spmm_fwd(a_dev[:T], vals, meta, N, K_BIG, Y=g.t)
    g.check("Y")
    gemm_full(g.t, a[:T], c["vals_row"], c["meta_row"], N, K_BIG, True, chunk=1024)


@pytest.mark.parametrize("T", [T_FAST, T_GENERIC])
def test_spmm_bwd_input_at_the_offset_limit(sp, big, forms, T):
    """dX = dY Ws for a [65472, 256] weight, whose column form [256, 32736] is
    given as the row form above (any valid 2:4 form is a valid operand)."""
    a, a_dev = big
    c, (vals, meta) = forms
    g = Guarded((T, N), torch.float16)
    sp.sp24_spmm_bwd_input(a_dev[:T], vals, meta, K_BIG, N, dX=g.t)
    g.check("dX")
    gemm_full(g.t, a[:T], c["vals_row"], c["meta_row"], K_BIG, N, False, chunk=1024)


def test_weight_grad_at_the_offset_limit(sp, big):
    """dW [65520, 16] = dY^T X over 16384 tokens: T*R just below 2^30."""
    a, a_dev = big
    T, R, C = 16384, 65520, 16
    assert T * R < 2 ** 30 <= T * (R + 16)
    dY = a.reshape(-1)[:T * R].reshape(T, R)
    dY_dev = a_dev.view(-1)[:T * R].view(T, R)
    X = WL.normal_f16(SEED, 3, (T, C))
    g = Guarded((R, C), torch.float32)
    sp.sp24_weight_grad(dY_dev, torch.from_numpy(X).cuda(), dW=g.t)
    g.check("dW")
    want = O.weight_grad(dY, X, None, None, 0.0)
    got = g.t.cpu().numpy().astype(np.float64)
    err = np.abs(got - want).max() / np.abs(want).max()
    assert err <= DW_MAX_REL, err
    # one more row of weights would take the token offsets past 32 bits
    with pytest.raises(sp.Sp24Error, match="TOO_LARGE"):
        sp.sp24_weight_grad(a_dev.view(-1)[:T * (R + 16)].view(T, R + 16), torch.from_numpy(X).cuda())
