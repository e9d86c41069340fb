"""A gated 2:4 FFN layer step (structured_sparse_transformer_amd/ffn.py),
composed from the entry points on the GPU, against the same composition in
the oracle on the same seeded inputs.

The oracle rounds to fp16 where the GPU path stores fp16 (the products U,
the GEGLU output, the hidden gradient and dU), so each stage sees inputs of
the same precision; the outputs are compared normwise, at the GEMM
tolerance, since fp32 accumulation order and ties at those roundings differ.
After a noisy update of both weights, the layer's flip counters must equal
the oracle's counts exactly.
"""
import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MAX_REL = 1e-2


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16)


def oracle_step(W1, W2, X, dY, decay):
    two_h, d = W1.shape
    h = two_h // 2
    i1, i2 = O.mask_search(W1), O.mask_search(W2)
    c1, c2 = O.compress(W1, i1), O.compress(W2, i2)
    U = f16(O.spmm_fwd(X, c1["vals_row"], c1["meta_row"], two_h, d))
    Hg = f16(O.geglu_fwd(U, 16))
    Y = O.spmm_fwd(Hg, c2["vals_row"], c2["meta_row"], d, h)
    dHg = f16(O.spmm_bwd_input(dY, c2["vals_col"], c2["meta_col"], d, h))
    dW2 = O.weight_grad(dY, Hg, W2, i2, decay)
    dU = f16(O.geglu_bwd(U, dHg, 16))
    dX = O.spmm_bwd_input(dU, c1["vals_col"], c1["meta_col"], two_h, d)
    dW1 = O.weight_grad(dU, X, W1, i1, decay)
    return {"Y": Y, "dX": dX, "dW1": dW1, "dW2": dW2}


@pytest.mark.parametrize("T,d,h", [(256, 128, 256), (1000, 512, 1024)])
def test_gated_ffn_step_matches_the_oracle(T, d, h):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd.ffn import SparseGegluFFN
    seed = T + d + h
    W1 = WL.normal_f16(seed, 1, (2 * h, d), 0.02)
    W2 = WL.normal_f16(seed, 2, (d, h), 0.02)
    X = WL.normal_f16(seed, 3, (T, d))
    dY = WL.normal_f16(seed, 4, (T, d))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    layer = SparseGegluFFN(dev(W1), dev(W2), decay=1e-2)
    layer.refresh()
    Y, saved = layer.forward(dev(X))
    dX, dW1, dW2 = layer.backward(dev(dY), saved)
    got = {"Y": Y, "dX": dX, "dW1": dW1, "dW2": dW2}
    want = oracle_step(W1, W2, X, dY, 1e-2)
    for k in want:
        g = got[k].float().cpu().numpy().astype(np.float64)
        assert g.shape == want[k].shape, k
        err = np.abs(g - want[k]).max() / np.abs(want[k]).max()
        assert err <= MAX_REL, (k, err)

    # a noisy update of both weights: the next refresh counts flipped entries
    W1n = (W1.astype(np.float32) + WL.noise_f32(seed, 1, W1.shape, 1e-3)).astype(np.float16)
    W2n = (W2.astype(np.float32) + WL.noise_f32(seed, 2, W2.shape, 1e-3)).astype(np.float16)
    layer.W1.copy_(dev(W1n))
    layer.W2.copy_(dev(W2n))
    layer.refresh()
    want_flips = [O.flip_count(O.mask_search(W1), O.mask_search(W1n)),
                  O.flip_count(O.mask_search(W2), O.mask_search(W2n))]
    assert layer.flips.cpu().tolist() == want_flips
