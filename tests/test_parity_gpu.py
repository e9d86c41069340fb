"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Masks, indices, compressed values and metadata must match the oracle bit for
bit (the library's forms are taken out of their blocked order first).  GEMM outputs (fp16 in, fp32 accumulation, fp16 out) must be within a
normwise max relative error of 1e-2 and a mean absolute error of 1e-3 of the
oracle's float64 product.  Full-size GEMMs are checked element by element
(the oracle runs over chunks of token rows), with the column-sum identity as
an extra check; the 1.5B noisy loop's middle steps compare 512 random token
rows per GEMM.  Guard bands around outputs catch writes outside them.  All inputs are seeded synthetic draws (structured_sparse_transformer_amd.workloads).
"""
import os

import numpy as np
import pytest

from oracle import sp24_oracle as O
from structured_sparse_transformer_amd import workloads as WL

from forms_layout import block_width, from_blocked
from gpu_checks import Guarded, check_all, gemm_full, guarded_forms

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
MAX_REL, MEAN_ABS = 1e-2, 1e-3
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_blocks.txt")


@pytest.fixture(scope="module")
def sp():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from structured_sparse_transformer_amd import sp24
    sp24.lib()          # raises if the library was not built
    return sp24


def dev(a: np.ndarray):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t, dtype=None):
    a = t.cpu().numpy()
    if dtype == np.uint16:
        a = a.view(np.uint16)
    return a


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16) if a.dtype == np.float16 else a


def assert_forms_equal(got: dict, want: dict):
    for k in ("vals_row", "meta_row", "vals_col", "meta_col"):
        if k not in got:
            continue
        g = from_blocked(host(got[k], np.uint16 if k.startswith("meta") else None), block_width(k))
        w = want[k]
        assert g.shape == w.shape, k
        bad = np.argwhere(bits(g) != bits(w))
        assert bad.size == 0, f"{k}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


def assert_idx_equal(got, want):
    g = host(got)
    bad = np.argwhere(g != want)
    assert bad.size == 0, f"idx: {len(bad)} mismatches, first {bad[:3].tolist()} got {g[tuple(bad[0])]} want {want[tuple(bad[0])]}"


def check_gemm(out, ref):
    mr, ma = O.gemm_errors(out.astype(np.float64), ref)
    assert mr <= MAX_REL and ma <= MEAN_ABS, (mr, ma)
    return mr, ma


def golden_blocks():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, idx, _score, _note = [t.strip() for t in line.split("|")]
            v = [float.fromhex(t) if "0x" in t else float(t) for t in vals.split()]
            rows.append((name, np.array(v, dtype=np.float16).reshape(4, 4), int(idx)))
    return rows


def wide_range_matrix(seed, R, C):
    """fp16 entries spanning subnormals to large normals, with zeros and +-0."""
    rng = np.random.default_rng(seed)
    e = rng.uniform(-24, 15.9, size=(R, C))
    v = np.sign(rng.standard_normal((R, C))) * np.exp2(e)
    v[rng.random((R, C)) < 0.1] = 0.0
    w = v.astype(np.float16)
    w[rng.random((R, C)) < 0.05] = np.float16(-0.0)
    return w


# ----------------------------------------------------------------------------
# mask search

def test_mask_search_tiny(sp):
    w1, _ = WL.ffn_weights(WL.TINY)
    assert_idx_equal(sp.sp24_mask_search(dev(w1)), O.mask_search(w1))


def test_mask_search_handworked_blocks(sp):
    g = golden_blocks()
    W = np.concatenate([b for _, b, _ in g], axis=1)            # [4, 4n]
    got = host(sp.sp24_mask_search(dev(W)))[0]
    assert got.tolist() == [i for _, _, i in g]
    # the same blocks through the fused kernel (padded to a 16 x 16k matrix)
    n = W.shape[1]
    Wp = np.zeros((16, ((n + 15) // 16) * 16), np.float16)
    Wp[:4, :n] = W
    o = sp.sp24_search_compress(dev(Wp))
    assert host(o["idx"])[0, : len(g)].tolist() == [i for _, _, i in g]
    assert_forms_equal(o, O.compress(Wp, O.mask_search(Wp)))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_mask_search_wide_dynamic_range(sp, seed):
    # most of these blocks are outside the fp32-exact regime: exercises the
    # row-major sequential path, subnormals and signed zeros
    W = wide_range_matrix(seed, 128, 256)
    assert_idx_equal(sp.sp24_mask_search(dev(W)), O.mask_search(W))
    o = sp.sp24_search_compress(dev(W))
    want_idx = O.mask_search(W)
    assert_idx_equal(o["idx"], want_idx)
    assert_forms_equal(o, O.compress(W, want_idx))


def test_mask_search_infinities(sp):
    W = wide_range_matrix(9, 64, 64)
    rng = np.random.default_rng(10)
    W[rng.random(W.shape) < 0.02] = np.float16(np.inf)
    W[rng.random(W.shape) < 0.02] = np.float16(-np.inf)
    W[0:4, 0:4] = np.float16(np.inf)
    assert_idx_equal(sp.sp24_mask_search(dev(W)), O.mask_search(W))


@pytest.mark.parametrize("shape", [(4, 4), (12, 20), (36, 52), (8, 1028), (1028, 8)])
def test_mask_search_ragged_shapes(sp, shape):
    W = (np.random.default_rng(shape[0] * 7 + shape[1]).standard_normal(shape) * 0.02).astype(np.float16)
    assert_idx_equal(sp.sp24_mask_search(dev(W)), O.mask_search(W))


def test_mask_search_empty(sp):
    assert tuple(sp.sp24_mask_search(torch.empty(0, 16, dtype=torch.float16, device="cuda")).shape) == (0, 4)


def test_stress_config_bit_exact(sp):
    W = WL.stress_weight(WL.STRESS_SEED)
    want = O.mask_search(W)
    d = dev(W)
    assert_idx_equal(sp.sp24_mask_search(d), want)
    o = sp.sp24_search_compress(d)
    assert_idx_equal(o["idx"], want)
    assert_forms_equal(o, O.compress(W, want))
    # blocks fully inside the all-equal band tie on every pattern -> index 0
    assert (want[2048 // 4: 2108 // 4] == 0).all()


# ----------------------------------------------------------------------------
# compression

@pytest.mark.parametrize("shape", [(16, 16), (144, 272), (272, 144), (128, 128), (256, 384)])
def test_compress_given_idx(sp, shape):
    W = (np.random.default_rng(shape[0] + 3 * shape[1]).standard_normal(shape) * 0.02).astype(np.float16)
    idx = O.mask_search(W)
    want = O.compress(W, idx)
    d = dev(W)
    assert_forms_equal(sp.sp24_compress(d, dev(idx)), want)
    assert_forms_equal(sp.sp24_compress(d, dev(idx), col=False), {k: want[k] for k in ("vals_row", "meta_row")})
    assert_forms_equal(sp.sp24_compress(d, dev(idx), row=False), {k: want[k] for k in ("vals_col", "meta_col")})
    o = sp.sp24_search_compress(d)
    assert_idx_equal(o["idx"], idx)
    assert_forms_equal(o, want)


def test_search_compress_batch(sp):
    # several weights, mixed shapes (with row and column tails), one launch
    shapes = [(144, 272), (272, 144), (16, 16), (512, 128), (64, 1040)]
    Ws = [(np.random.default_rng(40 + k).standard_normal(sh) * 0.02).astype(np.float16) for k, sh in enumerate(shapes)]
    Ws[1] = wide_range_matrix(45, 272, 144)            # exact-order path inside a batch
    outs = sp.sp24_search_compress_batch([dev(W) for W in Ws])
    for W, o in zip(Ws, outs):
        idx = O.mask_search(W)
        assert_idx_equal(o["idx"], idx)
        assert_forms_equal(o, O.compress(W, idx))


def test_search_compress_batch_ffn_pair(sp):
    w1, w2 = WL.ffn_weights(WL.GPT2_1P5B)
    o1, o2 = sp.sp24_search_compress_batch([dev(w1), dev(w2)])
    for W, o in ((w1, o1), (w2, o2)):
        idx = O.mask_search(W)
        assert_idx_equal(o["idx"], idx)
        assert_forms_equal(o, O.compress(W, idx))


def test_compress_random_indices(sp):
    # any index 0..89 per block, not only searched ones
    W = WL.normal_f16(77, 1, (64, 96), 1.0)
    idx = np.random.default_rng(78).integers(0, 90, size=(16, 24)).astype(np.uint8)
    assert_forms_equal(sp.sp24_compress(dev(W), dev(idx)), O.compress(W, idx))


def test_outputs_stay_inside_their_buffers(sp):
    R, C = 144, 272
    W = (np.random.default_rng(5).standard_normal((R, C)) * 0.02).astype(np.float16)
    pad = 4096                                    # guard bytes on each side (keeps 16-byte alignment)
    spec = {"idx": ((R // 4, C // 4), torch.uint8), "vals_row": ((R, C // 2), torch.float16),
            "meta_row": ((R, C // 16), torch.int16), "vals_col": ((C, R // 2), torch.float16),
            "meta_col": ((C, R // 16), torch.int16)}
    raw, views = {}, {}
    for k, (shape, dt) in spec.items():
        nbytes = int(np.prod(shape)) * torch.empty(0, dtype=dt).element_size()
        raw[k] = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
        views[k] = raw[k][pad: pad + nbytes].view(dt).view(shape)
    o = sp.sp24_search_compress(dev(W), out=views)
    torch.cuda.synchronize()
    for k, b in raw.items():
        h = b.cpu().numpy()
        assert (h[:pad] == 0xA5).all() and (h[-pad:] == 0xA5).all(), k
    idx = O.mask_search(W)
    assert_idx_equal(o["idx"], idx)
    assert_forms_equal(o, O.compress(W, idx))


# ----------------------------------------------------------------------------
# GEMMs

def _forms_dev(sp, W):
    o = sp.sp24_search_compress(dev(W))
    return o


def _gemm_pair(sp, W, X, dY):
    R, C = W.shape
    o = _forms_dev(sp, W)
    Y = sp.sp24_spmm_fwd(dev(X), o["vals_row"], o["meta_row"], R, C)
    dX = sp.sp24_spmm_bwd_input(dev(dY), o["vals_col"], o["meta_col"], R, C)
    return o, host(Y), host(dX)


def test_spmm_tiny(sp):
    inp = WL.ffn_inputs(WL.TINY)
    W = inp.w1
    R, C = W.shape
    o, Y, dX = _gemm_pair(sp, W, inp.x, inp.dy2)
    c = O.compress(W, O.mask_search(W))
    check_gemm(Y, O.spmm_fwd(inp.x, c["vals_row"], c["meta_row"], R, C))
    check_gemm(dX, O.spmm_bwd_input(inp.dy2, c["vals_col"], c["meta_col"], R, C))


@pytest.mark.parametrize("T,R,C", [(1, 16, 16), (7, 48, 80), (100, 272, 144), (129, 256, 512), (300, 528, 336),
                                   (256, 64, 4112), (300, 320, 192)])
def test_spmm_ragged(sp, T, R, C):
    rng = np.random.default_rng(T * 131 + R * 7 + C)
    W = (rng.standard_normal((R, C)) * 0.02).astype(np.float16)
    X = rng.standard_normal((T, C)).astype(np.float16)
    dY = rng.standard_normal((T, R)).astype(np.float16)
    o, Y, dX = _gemm_pair(sp, W, X, dY)
    c = O.compress(W, O.mask_search(W))
    check_gemm(Y, O.spmm_fwd(X, c["vals_row"], c["meta_row"], R, C))
    check_gemm(dX, O.spmm_bwd_input(dY, c["vals_col"], c["meta_col"], R, C))


def test_spmm_empty_tokens(sp):
    W = WL.normal_f16(3, 1, (32, 32), 0.02)
    o = _forms_dev(sp, W)
    Y = sp.sp24_spmm_fwd(torch.empty(0, 32, dtype=torch.float16, device="cuda"), o["vals_row"], o["meta_row"], 32, 32)
    assert tuple(Y.shape) == (0, 32)


def test_spmm_empty_reduction(sp):
    """A weight with no columns (fwd) or no rows (bwd): every output is an
    empty sum, +0, and the kernels read no operand."""
    T, N = 300, 48
    e = lambda *s, dt=torch.float16: torch.empty(*s, dtype=dt, device="cuda")  # noqa: E731
    Y = torch.full((T, N), float("nan"), dtype=torch.float16, device="cuda")
    sp.sp24_spmm_fwd(e(T, 0), e(N, 0), e(N, 0, dt=torch.int16), N, 0, Y=Y)
    dX = torch.full((T, N), float("nan"), dtype=torch.float16, device="cuda")
    sp.sp24_spmm_bwd_input(e(T, 0), e(N, 0), e(N, 0, dt=torch.int16), 0, N, dX=dX)
    for out in (Y, dX):
        assert (out.view(torch.int16) == 0).all()


def test_spmm_exact_small_integers(sp):
    # small integers: every product and sum is exact in fp32 and the results
    # fit fp16 exactly, so the GEMM must match the oracle exactly
    rng = np.random.default_rng(4)
    T, R, C = 96, 160, 192
    W = rng.integers(-3, 4, size=(R, C)).astype(np.float16)
    X = rng.integers(-2, 3, size=(T, C)).astype(np.float16)
    dY = rng.integers(-2, 3, size=(T, R)).astype(np.float16)
    o, Y, dX = _gemm_pair(sp, W, X, dY)
    c = O.compress(W, O.mask_search(W))
    assert (Y.astype(np.float64) == O.spmm_fwd(X, c["vals_row"], c["meta_row"], R, C)).all()
    assert (dX.astype(np.float64) == O.spmm_bwd_input(dY, c["vals_col"], c["meta_col"], R, C)).all()


def _sampled_rows(T, n, seed):
    return np.sort(np.random.default_rng(seed).choice(T, size=min(n, T), replace=False))


def check_full_gemm(out_dev, A, vals, meta, R, C, fwd: bool, seed: int):
    """Every element against the oracle (chunked over tokens), plus the
    column-sum identity over all rows as an extra check."""
    mr, ma = gemm_full(out_dev, A, vals, meta, R, C, fwd)
    # sum over tokens: sum_t out[t] = (sum_t A[t]) * Ws^T (fwd) or * Ws (bwd)
    colsum = out_dev.float().sum(dim=0).double().cpu().numpy()
    a_sum = A.astype(np.float64).sum(axis=0, keepdims=True)
    ref_sum = (O.spmm_fwd if fwd else O.spmm_bwd_input)(a_sum, vals, meta, R, C)[0]
    err = np.abs(colsum - ref_sum).max() / np.abs(ref_sum).max()
    assert err <= MAX_REL, err
    return mr, ma


@pytest.mark.parametrize("N", [1152, 1280, 6400])
def test_spmm_tail_split_ragged_tokens(sp, N):
    """Feature counts whose last 256-wide strip leaves a partial round on 256
    CUs run that strip as smaller tiles: 256 x 64 when 128 features remain
    (N = 1152), 128 x 128 when 256 remain (N = 1280, and the 6400 features of
    the GPT-2-1.5B FFN).  A ragged token count (16347, not a multiple of 64)
    puts rows past T into the last tiles of both launches.  Every element of
    both products is checked, with guard bands around each output: the strip
    launch writes at a column offset with the full row stride."""
    T, K = 16347, 128
    W = WL.normal_f16(N + 7, 1, (N, K), 0.02)
    X = WL.normal_f16(N + 7, 2, (T, K))
    Wt = WL.normal_f16(N + 7, 4, (K, N), 0.02)          # input gradient with N output features
    dY = WL.normal_f16(N + 7, 3, (T, K))
    c = O.compress(W, O.mask_search(W))
    ct = O.compress(Wt, O.mask_search(Wt))
    fw = guarded_forms(N, K)
    o = sp.sp24_search_compress(dev(W), out={k: g.t for k, g in fw.items()})
    bw = guarded_forms(K, N)
    ot = sp.sp24_search_compress(dev(Wt), out={k: g.t for k, g in bw.items()})
    assert_forms_equal(o, c)
    assert_forms_equal(ot, ct)
    gY, gdX = Guarded((T, N), torch.float16), Guarded((T, N), torch.float16)
    sp.sp24_spmm_fwd(dev(X), o["vals_row"], o["meta_row"], N, K, Y=gY.t)
    sp.sp24_spmm_bwd_input(dev(dY), ot["vals_col"], ot["meta_col"], K, N, dX=gdX.t)
    check_all(fw)
    check_all(bw)
    gY.check("Y")
    gdX.check("dX")
    check_full_gemm(gY.t, X, c["vals_row"], c["meta_row"], N, K, True, N)
    check_full_gemm(gdX.t, dY, ct["vals_col"], ct["meta_col"], K, N, False, N + 1)


@pytest.mark.parametrize("cfg", [WL.GPT2_355M, WL.GPT2_774M, WL.GPT2_1P5B], ids=lambda c: c.name)
def test_ffn_layer_configs(sp, cfg):
    """Search, compression and the four sparse GEMMs of a GPT-2 FFN layer at
    full size: masks and forms bit for bit, every GEMM output element against
    the oracle, guard bands around every output."""
    inp = WL.ffn_inputs(cfg)
    for which, W, A_fwd, A_bwd in ((1, inp.w1, inp.x, inp.dy1), (2, inp.w2, inp.h, inp.dy2)):
        R, C = W.shape
        T = A_fwd.shape[0]
        print(f"{cfg.name} W{which} {R}x{C}", flush=True)
        idx = O.mask_search(W)
        want = O.compress(W, idx)
        g = guarded_forms(R, C)
        o = sp.sp24_search_compress(dev(W), out={k: v.t for k, v in g.items()})
        gY, gdX = Guarded((T, R), torch.float16), Guarded((T, C), torch.float16)
        sp.sp24_spmm_fwd(dev(A_fwd), o["vals_row"], o["meta_row"], R, C, Y=gY.t)
        sp.sp24_spmm_bwd_input(dev(A_bwd), o["vals_col"], o["meta_col"], R, C, dX=gdX.t)
        check_all(g)
        gY.check("Y")
        gdX.check("dX")
        assert_idx_equal(o["idx"], idx)
        assert_forms_equal(o, want)
        check_full_gemm(gY.t, A_fwd, want["vals_row"], want["meta_row"], R, C, True, which)
        check_full_gemm(gdX.t, A_bwd, want["vals_col"], want["meta_col"], R, C, False, 10 + which)


@pytest.mark.parametrize("chunk", range(4))
def test_noisy_loop_1p5b(sp, chunk):
    """The 1.5B noisy loop (20 steps of W <- fp16(f32(W) + N(0, 1e-3))), in four
    chunks of five steps so that each test stays short.  At every step, for W1
    and W2: masks and both compressed forms bit-exact against the oracle, and
    from each chunk's second step on the fused flip counts against the previous
    step's masks.  The four GEMMs: sampled rows plus the column-sum identity over
    all tokens at steps 0 and 19, and 512 random token rows at every other step."""
    cfg = WL.GPT2_1P5B
    inp = WL.ffn_inputs(cfg)
    steps = cfg.steps
    per = steps // 4
    lo, hi = chunk * per, (chunk + 1) * per
    acts = {"X": (inp.x, dev(inp.x)), "H": (inp.h, dev(inp.h)), "dY1": (inp.dy1, dev(inp.dy1)),
            "dY2": (inp.dy2, dev(inp.dy2))}
    prev_dev, prev_host = None, None
    chain = zip(WL.noisy_weights(cfg, inp.w1, 1, steps), WL.noisy_weights(cfg, inp.w2, 2, steps))
    for (s, w1), (_, w2) in chain:
        if s < lo:
            continue
        if s >= hi:
            break
        print(f"noisy loop step {s}", flush=True)
        flips = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in range(2)]
        outs = sp.sp24_search_compress_batch(
            [dev(w1), dev(w2)], prev=prev_dev, flips=flips if prev_dev is not None else None)
        idx_host, forms = [], []
        for o, W in zip(outs, (w1, w2)):
            idx = O.mask_search(W)
            assert_idx_equal(o["idx"], idx)
            forms.append(O.compress(W, idx))
            assert_forms_equal(o, forms[-1])
            idx_host.append(idx)
        if prev_dev is not None:
            for f, a, b in zip(flips, prev_host, idx_host):
                assert int(f.item()) == O.flip_count(a, b), s
        # previous masks for the next step: copies, since the next launch writes new index buffers
        prev_dev = [o["idx"].clone() for o in outs]
        prev_host = idx_host
        (R1, C1), (R2, C2) = w1.shape, w2.shape
        o1, o2 = outs
        gemms = [  # (name, output, oracle operand, vals, meta, R, C, forward?)
            ("fwd1", sp.sp24_spmm_fwd(acts["X"][1], o1["vals_row"], o1["meta_row"], R1, C1), "X", "row", 0, R1, C1, True),
            ("bwd1", sp.sp24_spmm_bwd_input(acts["dY1"][1], o1["vals_col"], o1["meta_col"], R1, C1), "dY1", "col", 0, R1,
             C1, False),
            ("fwd2", sp.sp24_spmm_fwd(acts["H"][1], o2["vals_row"], o2["meta_row"], R2, C2), "H", "row", 1, R2, C2, True),
            ("bwd2", sp.sp24_spmm_bwd_input(acts["dY2"][1], o2["vals_col"], o2["meta_col"], R2, C2), "dY2", "col", 1, R2,
             C2, False),
        ]
        for name, out, a, form, k, R, C, fwd in gemms:
            A = acts[a][0]
            vals, meta = forms[k][f"vals_{form}"], forms[k][f"meta_{form}"]
            if s in (0, steps - 1):
                check_full_gemm(out, A, vals, meta, R, C, fwd, 100 * s + len(name))
            else:
                rows = _sampled_rows(A.shape[0], 512, 1000 * s + k * 10 + int(fwd))
                ref = (O.spmm_fwd if fwd else O.spmm_bwd_input)(A[rows], vals, meta, R, C)
                check_gemm(host(out[torch.from_numpy(rows).cuda()]), ref)
