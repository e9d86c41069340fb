"""GPU parity of the grouped sparse GEMM launch (sp24_spmm_group).

Each product of a group must equal the single-launch entry points'
(sp24_spmm_fwd / sp24_spmm_bwd_input) output bit for bit: both run the same
tile code with the same K order per output, and the single launches are
checked against the oracle elsewhere.  Here the grouped outputs are also
checked against the oracle element by element at the GPT-2-1.5B shapes,
inside guard bands, and the workspace must be all zero after every call
(the launch hands its queues back reset).
"""
import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

from forms_layout import META_BLOCK, VALS_BLOCK, from_blocked
from gpu_checks import Guarded, gemm_full

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


def workspace_is_zero(sp):
    torch.cuda.synchronize()
    return bool((sp.group_workspace() == 0).all())


def ffn_products(sp, cfg, tokens=None):
    """The four products of one FFN layer step: (name, A, vals, meta, R, C, fwd)."""
    inp = WL.ffn_inputs(cfg, tokens)
    f1 = sp.sp24_search_compress(dev(inp.w1))
    f2 = sp.sp24_search_compress(dev(inp.w2))
    (R1, C1), (R2, C2) = inp.w1.shape, inp.w2.shape
    return inp, [
        ("fwd1", inp.x, f1["vals_row"], f1["meta_row"], R1, C1, True),
        ("bwd1", inp.dy1, f1["vals_col"], f1["meta_col"], R1, C1, False),
        ("fwd2", inp.h, f2["vals_row"], f2["meta_row"], R2, C2, True),
        ("bwd2", inp.dy2, f2["vals_col"], f2["meta_col"], R2, C2, False),
    ]


def single(sp, A_dev, vals, meta, R, C, fwd):
    if fwd:
        return sp.sp24_spmm_fwd(A_dev, vals, meta, R, C)
    return sp.sp24_spmm_bwd_input(A_dev, vals, meta, R, C)


@pytest.mark.parametrize("cfg", [WL.GPT2_355M, WL.GPT2_1P5B], ids=lambda c: c.name)
def test_group_equals_single_launches(sp, cfg):
    """The four GEMMs of an FFN layer step in one launch, twice in a row (the
    second call runs on the queues the first one reset): bit-identical to the
    single launches, nothing written outside the outputs."""
    inp, prods = ffn_products(sp, cfg)
    acts = [dev(p[1]) for p in prods]
    want = [single(sp, a, v, m, R, C, fwd) for a, (_, _, v, m, R, C, fwd) in zip(acts, prods)]
    for call in range(2):
        guards = [Guarded(w.shape, torch.float16) for w in want]
        sp.sp24_spmm_group([(a, v, m, g.t) for a, (_, _, v, m, _, _, _), g in zip(acts, prods, guards)])
        for (name, *_), g, w in zip(prods, guards, want):
            g.check(f"{name} call {call}")
            assert torch.equal(g.t, w), f"{name} call {call}"
        assert workspace_is_zero(sp)


def test_group_gpt2_1p5b_against_the_oracle(sp):
    """Every element of the four grouped products of the 1.5B layer against
    the oracle's float64 products."""
    cfg = WL.GPT2_1P5B
    inp, prods = ffn_products(sp, cfg)
    outs = sp.sp24_spmm_group([(dev(A), v, m, None) for _, A, v, m, _, _, _ in prods])
    for (name, A, v, m, R, C, fwd), out in zip(prods, outs):
        print(f"group {name}", flush=True)
        vals = from_blocked(v.cpu().numpy(), VALS_BLOCK)
        meta = from_blocked(m.cpu().numpy().view(np.uint16), META_BLOCK)
        gemm_full(out, A, vals, meta, R, C, fwd)


def test_group_mixed_shapes(sp):
    """A group with a product the persistent kernel does not take (K = 80, run
    as a single launch), an empty product, ragged token and feature counts and
    K = 192 (three stages, the smallest the kernel takes); and a lone product."""
    rng = np.random.default_rng(5)
    shapes = [(300, 272, 192), (37, 48, 80), (0, 64, 128), (513, 528, 256), (1000, 1040, 448)]
    prods, want = [], []
    for T, N, K in shapes:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        A = rng.standard_normal((T, K)).astype(np.float16)
        f = sp.sp24_search_compress(dev(W))
        prods.append((dev(A), f["vals_row"], f["meta_row"]))
        want.append(sp.sp24_spmm_fwd(prods[-1][0], f["vals_row"], f["meta_row"], N, K))
        c = O.compress(W, O.mask_search(W))
        if T:
            gemm_full(want[-1], A, c["vals_row"], c["meta_row"], N, K, True)
    guards = [Guarded((T, N), torch.float16) for T, N, _ in shapes]
    sp.sp24_spmm_group([(a, v, m, g.t) for (a, v, m), g in zip(prods, guards)])
    for k, (g, w) in enumerate(zip(guards, want)):
        g.check(f"product {k}")
        assert torch.equal(g.t, w), k
    assert workspace_is_zero(sp)
    lone = sp.sp24_spmm_group([prods[-1] + (None,)])[0]
    assert torch.equal(lone, want[-1])
    assert workspace_is_zero(sp)


def test_group_workspace_of_the_caller(sp):
    """A caller-supplied workspace (zeroed) works like the binding's and is
    handed back zeroed; the binding refuses one that is too small."""
    _, prods = ffn_products(sp, WL.GPT2_355M, tokens=2048)
    ws = torch.zeros(16, dtype=torch.int32, device="cuda")
    outs = sp.sp24_spmm_group([(dev(A), v, m, None) for _, A, v, m, _, _, _ in prods], workspace=ws)
    torch.cuda.synchronize()
    assert (ws == 0).all()
    for (_, A, v, m, R, C, fwd), out in zip(prods, outs):
        assert torch.equal(out, single(sp, dev(A), v, m, R, C, fwd))
    with pytest.raises(ValueError):
        sp.sp24_spmm_group([(dev(prods[0][1]), prods[0][2], prods[0][3], None)], workspace=ws[:8])
