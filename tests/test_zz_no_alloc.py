"""The allocation-free grouped GEMM entry point (sp24_spmm_group_noalloc)
against sp24_spmm_group, through the C ABI: bit-identical outputs on two calls
in a row, the second with smaller products, every output pre-allocated so the
calls themselves allocate nothing."""
import numpy as np
import pytest

from structured_sparse_transformer_amd import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sp():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd import sp24
    sp24.lib()
    return sp24


def step_products(sp, cfg, tokens):
    inp = WL.ffn_inputs(cfg, tokens)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    f1 = sp.sp24_search_compress(dev(inp.w1))
    f2 = sp.sp24_search_compress(dev(inp.w2))
    return [(dev(inp.x), f1["vals_row"], f1["meta_row"]), (dev(inp.dy1), f1["vals_col"], f1["meta_col"]),
            (dev(inp.h), f2["vals_row"], f2["meta_row"]), (dev(inp.dy2), f2["vals_col"], f2["meta_col"])]


def outputs_for(prods):
    return [torch.full((A.shape[0], v.shape[0]), float("nan"), dtype=torch.float16, device="cuda")
            for A, v, _ in prods]


@pytest.mark.parametrize("first,second", [((WL.GPT2_1P5B, 16384), (WL.GPT2_355M, 4096))],
                         ids=["1.5b-then-smaller"])
def test_noalloc_matches_the_workspace_entry_point(sp, first, second):
    for cfg, tokens in (first, second):
        prods = step_products(sp, cfg, tokens)
        want = sp.sp24_spmm_group([p + (o,) for p, o in zip(prods, outputs_for(prods))])
        got = outputs_for(prods)
        torch.cuda.synchronize()
        sp.sp24_spmm_group_noalloc([p + (o,) for p, o in zip(prods, got)])
        torch.cuda.synchronize()
        for k, (g, w) in enumerate(zip(got, want)):
            assert torch.equal(g, w), f"{cfg.name} product {k}"
    # and once more on the first shapes: the library's counters were handed
    # back reset by the calls above
    prods = step_products(sp, first[0], 2048)
    want = sp.sp24_spmm_group([p + (None,) for p in prods])
    got = sp.sp24_spmm_group_noalloc([p + (None,) for p in prods])
    for g, w in zip(got, want):
        assert torch.equal(g, w)


def test_noalloc_rejects_too_many_products(sp):
    prods = step_products(sp, WL.GPT2_355M, 256)
    with pytest.raises(ValueError):
        sp.sp24_spmm_group_noalloc([prods[0] + (None,)] * 9)
