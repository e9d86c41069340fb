"""GPU parity of the flip count (mask entries changed between two searches).

The oracle's flip_count is compared exactly (an integer) with the library's
standalone sp24_flip_count and with the count fused into the batched search.
Expected counts come from masks the oracle searched itself; the HIP path's
indices are never fed to the oracle.  Indices >= 90 are read as pattern 0 by
the library; the tests map them the same way before asking the oracle.
"""
import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL
from forms_layout import META_BLOCK, from_blocked

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


def counter(n=1):
    return torch.zeros(n, dtype=torch.int64, device="cuda")


def clamp90(a):
    return np.where(a < 90, a, 0).astype(np.uint8)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 4096 + 5, 640000, 1_000_003])
def test_flip_count_standalone(sp, n):
    a = WL.random_idx(7, 1, (n,))
    b = WL.random_idx(7, 2, (n,))
    got = sp.sp24_flip_count(dev(a), dev(b))
    assert int(got.item()) == O.flip_count(a, b)


def test_flip_count_identical_and_out_of_range(sp):
    a = WL.random_idx(8, 1, (5000,), hi=256)        # about 65% of entries >= 90
    b = WL.random_idx(8, 2, (5000,), hi=256)
    assert int(sp.sp24_flip_count(dev(a), dev(a)).item()) == 0
    got = sp.sp24_flip_count(dev(a), dev(b))
    assert int(got.item()) == O.flip_count(clamp90(a), clamp90(b))


def test_flip_count_adds(sp):
    a, b = WL.random_idx(9, 1, (3000,)), WL.random_idx(9, 2, (3000,))
    f = counter()
    f.fill_(12345)
    sp.sp24_flip_count(dev(a), dev(b), f)
    sp.sp24_flip_count(dev(b), dev(a), f)
    assert int(f.item()) == 12345 + 2 * O.flip_count(a, b)


def test_flip_count_empty(sp):
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    assert int(sp.sp24_flip_count(e, e).item()) == 0


def _two_steps(seed, R, C, which=1):
    w0 = WL.normal_f16(seed, 1, (R, C), WL.W_SIGMA)
    w1 = WL.add_noise_f16(w0, WL.noise_f32(seed * 10 + which, 0, (R, C), 3e-3))
    return w0, w1


@pytest.mark.parametrize("shape", [(16, 16), (144, 272), (272, 144), (256, 384), (1040, 656)])
def test_fused_flips_match_oracle(sp, shape):
    R, C = shape
    w0, w1 = _two_steps(40 + R, R, C)
    i0, i1 = O.mask_search(w0), O.mask_search(w1)
    want = O.flip_count(i0, i1)
    assert want > 0
    f = counter()
    o = sp.sp24_search_compress_batch([dev(w1)], prev=[dev(i0)], flips=[f[0:1]])[0]
    assert int(f.item()) == want
    assert (o["idx"].cpu().numpy() == i1).all()


def test_fused_flips_in_place(sp):
    """idx_prev is the job's own idx buffer: old masks read, new ones written."""
    R, C = 528, 784
    w0, w1 = _two_steps(77, R, C)
    i0, i1 = O.mask_search(w0), O.mask_search(w1)
    buf = dev(i0)
    f = counter()
    o = sp.sp24_search_compress_batch([dev(w1)], outs=[{"idx": buf}], prev=[buf], flips=[f])[0]
    assert o["idx"].data_ptr() == buf.data_ptr()
    assert int(f.item()) == O.flip_count(i0, i1)
    assert (buf.cpu().numpy() == i1).all()
    c = O.compress(w1, i1)
    assert (from_blocked(o["meta_row"].cpu().numpy().view(np.uint16), META_BLOCK) == c["meta_row"]).all()
    assert (from_blocked(o["meta_col"].cpu().numpy().view(np.uint16), META_BLOCK) == c["meta_col"]).all()


def test_fused_flips_shared_counter_and_bad_prev(sp):
    """Several jobs may add into one counter; previous indices >= 90 read as 0."""
    wa0, wa1 = _two_steps(91, 256, 128, 1)
    wb0, wb1 = _two_steps(92, 128, 400, 2)
    pa = O.mask_search(wa0)
    pb = np.full((32, 100), 0xFF, np.uint8)
    pb[::3] = O.mask_search(wb0)[::3]
    f = counter(2)
    f[0] = 7
    sp.sp24_search_compress_batch([dev(wa1), dev(wb1)], prev=[dev(pa), dev(pb)], flips=[f[0:1], f[0:1]])
    want = 7 + O.flip_count(pa, O.mask_search(wa1)) + O.flip_count(clamp90(pb), O.mask_search(wb1))
    assert int(f[0].item()) == want and int(f[1].item()) == 0


def test_fused_flips_without_idx_output(sp):
    R, C = 128, 256
    w0, w1 = _two_steps(93, R, C)
    i0 = O.mask_search(w0)
    f = counter()
    o = sp.sp24_search_compress_batch([dev(w1)], want_idx=False, prev=[dev(i0)], flips=[f])[0]
    assert "idx" not in o
    assert int(f.item()) == O.flip_count(i0, O.mask_search(w1))


def test_fused_flips_noisy_loop_355m(sp):
    """The noisy weight loop on one GPT-2 355M FFN layer: every step's fused
    count for both weights, in place, against the oracle's own searches."""
    cfg, steps = WL.GPT2_355M, 6
    w1, w2 = WL.ffn_weights(cfg)
    prev = [O.mask_search(w1), O.mask_search(w2)]
    bufs = [dev(prev[0]), dev(prev[1])]
    f = counter(2 * steps)
    for (s, a), (_, b) in zip(WL.noisy_weights(cfg, w1, 1, steps), WL.noisy_weights(cfg, w2, 2, steps)):
        sp.sp24_search_compress_batch([dev(a), dev(b)], outs=[{"idx": bufs[0]}, {"idx": bufs[1]}], prev=bufs,
                                      flips=[f[2 * s: 2 * s + 1], f[2 * s + 1: 2 * s + 2]])
        cur = [O.mask_search(a), O.mask_search(b)]
        got = f[2 * s: 2 * s + 2].cpu().numpy()
        want = [O.flip_count(prev[0], cur[0]), O.flip_count(prev[1], cur[1])]
        assert got.tolist() == want, s
        assert 0 < want[0] < a.size
        prev = cur


def test_fused_flips_1p5b_first_and_last_steps(sp):
    """GPT-2 1.5B FFN layer, 20-step noisy loop: fused counts at steps 1 and 19
    against the oracle; every other step's count is even and within range."""
    cfg = WL.GPT2_1P5B
    w1, w2 = WL.ffn_weights(cfg)
    steps = cfg.steps
    bufs = None
    f = counter(2 * steps)
    keep = {}
    for (s, a), (_, b) in zip(WL.noisy_weights(cfg, w1, 1, steps), WL.noisy_weights(cfg, w2, 2, steps)):
        if bufs is None:
            o = sp.sp24_search_compress_batch([dev(a), dev(b)])
            bufs = [o[0]["idx"], o[1]["idx"]]
        else:
            sp.sp24_search_compress_batch([dev(a), dev(b)], outs=[{"idx": bufs[0]}, {"idx": bufs[1]}], prev=bufs,
                                          flips=[f[2 * s: 2 * s + 1], f[2 * s + 1: 2 * s + 2]])
        if s in (0, 1, steps - 2, steps - 1):
            keep[s] = (a, b)
    got = f.cpu().numpy().reshape(steps, 2)
    for s in (1, steps - 1):
        for k in range(2):
            want = O.flip_count(O.mask_search(keep[s - 1][k]), O.mask_search(keep[s][k]))
            assert got[s, k] == want, (s, k)
    n = w1.size
    assert (got[1:] % 2 == 0).all() and (got[1:] > 0).all() and (got[1:] < n).all()
    assert (got[0] == 0).all()
