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


def test_gated_ffn_step_full_size_sampled():
    """The layer step at the size the bench times it (16384 tokens, W1 6400 x 1600
    read as h = 3200, W2 1600 x 3200), checked on samples the oracle computes
    cheaply: 32 token rows of Y and dX, and 8 x 8 entries of each weight
    gradient, from whole columns of U, Hg, dHg and dU over all tokens."""
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd.ffn import SparseGegluFFN
    T, d, h, decay, seed = 16384, 1600, 3200, 2e-4, 4242
    W1 = WL.normal_f16(seed, 1, (2 * h, d), 0.02)
    W2 = WL.normal_f16(seed, 2, (d, h), 0.02)
    X = WL.normal_f16(seed, 3, (T, d))
    dY = WL.normal_f16(seed, 4, (T, d))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    layer = SparseGegluFFN(dev(W1), dev(W2), decay=decay)
    layer.refresh()
    Y, saved = layer.forward(dev(X))
    dX, dW1, dW2 = layer.backward(dev(dY), saved)
    torch.cuda.synchronize()

    i1, i2 = O.mask_search(W1), O.mask_search(W2)
    c1, c2 = O.compress(W1, i1), O.compress(W2, i2)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(T, 32, replace=False))
    units = np.sort(rng.choice(h, 8, replace=False))       # hidden units (columns of Hg, W2)
    feats = np.sort(rng.choice(d, 8, replace=False))       # model features (columns of X, rows of W2)

    def unit_cols(u):
        # U columns of hidden unit u in blocks of 16 values then 16 gates: (value, gate)
        v = 32 * (u // 16) + u % 16
        return v, v + 16

    # token rows: the oracle composition on 32 rows
    U_s = f16(O.spmm_fwd(X[toks], c1["vals_row"], c1["meta_row"], 2 * h, d))
    Hg_s = f16(O.geglu_fwd(U_s, 16))
    Y_s = O.spmm_fwd(Hg_s, c2["vals_row"], c2["meta_row"], d, h)
    dHg_s = f16(O.spmm_bwd_input(dY[toks], c2["vals_col"], c2["meta_col"], d, h))
    dU_s = f16(O.geglu_bwd(U_s, dHg_s, 16))
    dX_s = O.spmm_bwd_input(dU_s, c1["vals_col"], c1["meta_col"], 2 * h, d)

    # whole columns for the sampled units: U's value and gate columns (rows of
    # the row form of W1), Hg, dHg (rows of the column form of W2) and dU
    Hg_u, dU_u, urows = [], [], []
    for u in units:
        vg = np.array(unit_cols(u))
        U_vg = f16(O.spmm_fwd(X, c1["vals_row"][vg], c1["meta_row"][vg], 2, d))
        Hg_u.append(f16(O.geglu_fwd(U_vg, 1))[:, 0])
        dHg_u = f16(O.spmm_bwd_input(dY, c2["vals_col"][[u]], c2["meta_col"][[u]], d, 1))
        dU_u.append(f16(O.geglu_bwd(U_vg, dHg_u, 1)))          # [T, 2]: d value, d gate
        urows.extend(vg)
    Hg_u = np.stack(Hg_u, axis=1)
    dU_u = np.concatenate(dU_u, axis=1)
    urows = np.array(urows)
    # decay terms of both weights, from the oracle with no tokens
    dec1 = O.weight_grad(np.zeros((0, 2 * h), np.float16), np.zeros((0, d), np.float16), W1, i1, decay)
    dec2 = O.weight_grad(np.zeros((0, d), np.float16), np.zeros((0, h), np.float16), W2, i2, decay)
    dW2_s = O.weight_grad(dY[:, feats], Hg_u, None, None, 0.0) + dec2[np.ix_(feats, units)]
    dW1_s = O.weight_grad(dU_u, X[:, feats], None, None, 0.0) + dec1[np.ix_(urows, feats)]

    got = {"Y": Y[toks].float().cpu().numpy(), "dX": dX[toks].float().cpu().numpy(),
           "dW1": dW1.cpu().numpy()[np.ix_(urows, feats)], "dW2": dW2.cpu().numpy()[np.ix_(feats, units)]}
    want = {"Y": Y_s, "dX": dX_s, "dW1": dW1_s, "dW2": dW2_s}
    for k in want:
        g = got[k].astype(np.float64)
        err = np.abs(g - want[k]).max() / np.abs(want[k]).max()
        assert err <= MAX_REL, (k, err)
