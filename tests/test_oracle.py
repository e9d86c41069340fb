"""Pins for the CPU oracle, checked against mathematics rather than itself.

Every test here runs on the CPU.  The oracle is pinned by:
* brute-force enumeration of all 2^16 4x4 0/1 masks (the pattern set and its
  known size, 90);
* exact rational scoring (``fractions.Fraction``) of random blocks whose
  sums are exact in fp32, compared with the oracle including the tie-break;
* hand-worked blocks in ``tests/golden/handworked_blocks.txt``;
* metamorphic properties (sign flips, power-of-two scaling, transposition,
  separable blocks, planted patterns);
* Algorithm 1 ("Accelerating Transformer Pre-training with 2:4 Sparsity")
  restated as one float64 matrix product of the flattened 4x4 blocks with
  the flattened patterns, and numpy's first-maximum argmax;
* for the GEMMs, an explicit float64 loop over the compressed storage and
  identity-matrix special cases.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import sp24_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_blocks.txt")


# ----------------------------------------------------------------------------
# brute-force reference for the pattern set (independent of the oracle's
# row-pair enumeration): every 16-bit mask, bit 4r+c for entry (r, c)
def _brute_patterns():
    pats = []
    for bits in range(1 << 16):
        m = np.array([(bits >> k) & 1 for k in range(16)], dtype=np.uint8).reshape(4, 4)
        if (m.sum(axis=0) == 2).all() and (m.sum(axis=1) == 2).all():
            pats.append(m)
    return pats


def _msb_first_key(m):
    """The 16-bit string of m read row by row, leftmost column first."""
    return int("".join(str(int(v)) for v in m.reshape(-1)), 2)


BRUTE = _brute_patterns()
# Pattern order pin: lexicographic over row-pair codes equals descending order
# of the row-major, leftmost-first bit string (code 0 = 1100 is the largest
# row string, code 5 = 0011 the smallest).
BRUTE_ORDERED = sorted(BRUTE, key=_msb_first_key, reverse=True)


def test_pattern_count_is_90():
    # The number of 4x4 0/1 matrices with all row and column sums 2 is 90.
    assert len(BRUTE) == 90
    assert len(O.pattern_codes()) == 90


def test_pattern_set_and_order_match_brute_force():
    masks = O.pattern_masks()
    assert masks.shape == (90, 4, 4)
    for p in range(90):
        assert (masks[p] == BRUTE_ORDERED[p]).all(), p
    # first and last patterns written out by hand
    assert masks[0].tolist() == [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]
    assert masks[89].tolist() == [[0, 0, 1, 1], [0, 0, 1, 1], [1, 1, 0, 0], [1, 1, 0, 0]]
    assert masks[23].tolist() == [[1, 0, 1, 0], [0, 1, 0, 1], [1, 0, 1, 0], [0, 1, 0, 1]]


def test_pattern_set_closed_under_transpose():
    keys = {m.tobytes() for m in O.pattern_masks()}
    for m in O.pattern_masks():
        assert np.ascontiguousarray(m.T).tobytes() in keys


# ----------------------------------------------------------------------------
# exact rational brute force of the mask search on one block
def _brute_block(block16):
    """(index, exact score) of the first maximum over BRUTE_ORDERED."""
    a = [Fraction(float(abs(v))) for v in np.asarray(block16, dtype=np.float16).reshape(-1)]
    best, best_s = None, None
    for p, m in enumerate(BRUTE_ORDERED):
        s = sum((a[k] for k in range(16) if m.reshape(-1)[k]), Fraction(0))
        if best is None or s > best_s:
            best, best_s = p, s
    return best, best_s


def _exact_regime(block16):
    """True when every partial sum of up to 8 entries is exact in fp32."""
    a = [Fraction(float(abs(v))) for v in np.asarray(block16, dtype=np.float16).reshape(-1)]
    nz = [x for x in a if x != 0]
    if not nz:
        return True
    # q = the finest power of two all entries are integer multiples of
    q = Fraction(1, 1 << 24)
    while all((x / (q * 2)).denominator == 1 for x in nz) and q < 2**20:
        q *= 2
    return 8 * max(a) < q * 2**24


def _random_blocks(rng, n, kind):
    if kind == "normal":
        b = (rng.standard_normal((n, 16)) * 0.02).astype(np.float16)
    elif kind == "ints":
        b = (rng.integers(-3, 4, size=(n, 16)) / 8).astype(np.float16)
    elif kind == "small-ints":
        b = rng.integers(-2, 3, size=(n, 16)).astype(np.float16)
    else:
        raise ValueError(kind)
    return b


@pytest.mark.parametrize("kind", ["normal", "ints", "small-ints"])
def test_mask_search_matches_exact_brute_force(kind):
    rng = np.random.default_rng([7, len(kind)])
    blocks = _random_blocks(rng, 300, kind)
    # lay the blocks out as a [4, 4*n] matrix: block j at columns 4j..4j+3
    W = blocks.reshape(-1, 4, 4).transpose(1, 0, 2).reshape(4, -1)
    idx = O.mask_search(W)[0]
    scores = O.block_scores(W)[0]
    for j, b in enumerate(blocks):
        assert _exact_regime(b)
        p, s = _brute_block(b)
        assert idx[j] == p, (j, b.reshape(4, 4))
        assert Fraction(float(scores[j, p])) == s


def _load_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, idx, score, _note = [t.strip() for t in line.split("|")]
            v = [float.fromhex(t) if "0x" in t else float(t) for t in vals.split()]
            rows.append((name, np.array(v, dtype=np.float16).reshape(4, 4), int(idx), float(score)))
    return rows


GOLDEN_ROWS = _load_golden()


@pytest.mark.parametrize("name,block,idx,score", GOLDEN_ROWS, ids=[r[0] for r in GOLDEN_ROWS])
def test_handworked_blocks(name, block, idx, score):
    assert O.mask_search(block)[0, 0] == idx
    assert float(O.block_scores(block)[0, 0, idx]) == score
    if _exact_regime(block):
        assert _brute_block(block)[0] == idx


def test_b7_b8_outside_exact_regime():
    g = {r[0]: r for r in GOLDEN_ROWS}
    b7, b8 = g["B7"][1], g["B8"][1]
    assert not _exact_regime(b7) and not _exact_regime(b8)
    # B7: the exact scores of 63 and 65 tie, so exact arithmetic also gives 63
    assert _brute_block(b7)[0] == 63
    # B8: exact arithmetic picks 24, fp32 in row-major order picks 11
    assert _brute_block(b8)[0] == 24
    assert O.mask_search(b8)[0, 0] == 11
    # B9: exact arithmetic picks 60, row-major fp32 picks 30
    b9 = g["B9"][1]
    assert not _exact_regime(b9)
    assert _brute_block(b9)[0] == 60
    assert O.mask_search(b9)[0, 0] == 30


# ----------------------------------------------------------------------------
# invariants and metamorphic properties on whole matrices
def _w(seed, R, C, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return (rng.standard_normal((R, C)) * 0.02).astype(np.float16)
    return (rng.integers(-3, 4, size=(R, C)) / 8).astype(np.float16)


@pytest.mark.parametrize("kind", ["normal", "ints"])
def test_mask_invariants(kind):
    W = _w(11, 64, 96, kind)
    idx = O.mask_search(W)
    assert idx.shape == (16, 24) and idx.dtype == np.uint8 and (idx < 90).all()
    M = O.idx_to_mask(idx)
    blocks = M.reshape(16, 4, 24, 4)
    assert (blocks.sum(axis=3) == 2).all()   # each block row keeps 2
    assert (blocks.sum(axis=1) == 2).all()   # each block column keeps 2


def test_sign_flips_do_not_change_mask():
    W = _w(12, 32, 32, "ints")
    rng = np.random.default_rng(5)
    sign = np.where(rng.random(W.shape) < 0.5, -1, 1).astype(np.float16)
    assert (O.mask_search(W) == O.mask_search(W * sign)).all()


@pytest.mark.parametrize("k", [-6, -1, 1, 5])
def test_power_of_two_scaling_does_not_change_mask(k):
    W = _w(13, 32, 64, "ints")
    W2 = (W.astype(np.float32) * np.float32(2.0 ** k)).astype(np.float16)
    assert (W2.astype(np.float32) == W.astype(np.float32) * 2.0 ** k).all()
    assert (O.mask_search(W) == O.mask_search(W2)).all()


def test_transpose_keeps_best_score():
    W = _w(14, 32, 32, "normal")
    s = O.block_scores(W).max(axis=2)
    st = O.block_scores(np.ascontiguousarray(W.T)).max(axis=2)
    assert (s == st.T).all()


def test_separable_blocks_tie_to_index_0():
    rng = np.random.default_rng(15)
    for _ in range(20):
        r = rng.integers(0, 8, size=(4, 1))
        c = rng.integers(0, 8, size=(1, 4))
        b = (r + c).astype(np.float16)
        assert O.mask_search(b)[0, 0] == 0


def test_planted_pattern_wins():
    masks = O.pattern_masks()
    for p in range(90):
        b = np.where(masks[p] == 1, 1.0, 0.25).astype(np.float16)
        assert O.mask_search(b)[0, 0] == p


def test_shape_rules():
    with pytest.raises(ValueError):
        O.mask_search(np.zeros((6, 8), np.float16))
    with pytest.raises(ValueError):
        O.compress(np.zeros((8, 8), np.float16), np.zeros((2, 2), np.uint8))
    with pytest.raises(TypeError):
        O.mask_search(np.zeros((8, 8), np.float32))


# ----------------------------------------------------------------------------
# Algorithm 1 of "Accelerating Transformer Pre-training with 2:4 Sparsity"
# (reproducibility table, Pseudocode row) scores every 4x4 block of
# |W| against every pattern (a correlation with stride 4 and no padding) and
# keeps the best pattern per block.  The same scores as one float64 matrix
# product: each block's 16 magnitudes, flattened row-major, against the 90
# patterns flattened the same way.
def test_blockwise_matmul_formulation():
    W = np.concatenate([_w(16, 32, 64, "normal"), _w(17, 32, 64, "ints")], axis=0)
    R, C = W.shape
    mags = np.abs(W.astype(np.float64))
    blocks = mags.reshape(R // 4, 4, C // 4, 4).transpose(0, 2, 1, 3).reshape(-1, 16)
    patterns = O.pattern_masks().reshape(90, 16).astype(np.float64)
    scores = blocks @ patterns.T                                     # [blocks, 90]
    best = np.argmax(scores, axis=1).reshape(R // 4, C // 4)         # numpy returns the first maximum
    assert (best == O.mask_search(W)).all()
    # in this (exact) regime the fp32 row-major scores equal the float64 products
    assert (O.block_scores(W).astype(np.float64).reshape(-1, 90) == scores).all()


# ----------------------------------------------------------------------------
# compression
def _decode_loop(vals, meta, n, m):
    """Explicit per-entry decode of one compressed form (rows of length m)."""
    out = np.zeros((n, m), dtype=np.float16)
    for i in range(n):
        for g in range(m // 4):
            nib = (int(meta[i, g // 4]) >> (4 * (g % 4))) & 0xF
            out[i, 4 * g + (nib & 3)] = vals[i, 2 * g]
            out[i, 4 * g + (nib >> 2)] = vals[i, 2 * g + 1]
    return out


@pytest.mark.parametrize("kind", ["normal", "ints"])
def test_compress_roundtrip(kind):
    W = _w(18, 48, 32, kind)
    W[0, 0] = np.float16(-0.0)
    idx = O.mask_search(W)
    c = O.compress(W, idx)
    R, C = W.shape
    assert c["vals_row"].shape == (R, C // 2) and c["meta_row"].shape == (R, C // 16)
    assert c["vals_col"].shape == (C, R // 2) and c["meta_col"].shape == (C, R // 16)
    M = O.idx_to_mask(idx)
    pruned = np.where(M, W, np.float16(0))
    d_row = O.decode_row_form(c["vals_row"], c["meta_row"], R, C)
    d_col = O.decode_col_form(c["vals_col"], c["meta_col"], R, C)
    assert (d_row.view(np.uint16) == pruned.view(np.uint16)).all()
    assert (d_col.view(np.uint16) == pruned.view(np.uint16)).all()
    assert (_decode_loop(c["vals_row"], c["meta_row"], R, C).view(np.uint16) == pruned.view(np.uint16)).all()
    assert (_decode_loop(c["vals_col"], c["meta_col"], C, R).T.view(np.uint16) == pruned.view(np.uint16)).all()
    legal = {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}
    for meta in (c["meta_row"], c["meta_col"]):
        for sh in (0, 4, 8, 12):
            assert set(np.unique((meta >> sh) & 0xF).tolist()) <= legal
    # kept values are stored in increasing in-group position, sign and all
    assert c["vals_row"].dtype == np.float16


def test_compress_worked_example_b3():
    # 16x16 tiling of the separable block 4r+c+1 -> every block picks pattern 0
    b = (np.arange(16, dtype=np.float32) + 1).reshape(4, 4)
    W = np.tile(b, (4, 4)).astype(np.float16)
    idx = O.mask_search(W)
    assert (idx == 0).all()
    c = O.compress(W, idx)
    # pattern 0 keeps columns {0,1} in rows 0,1 (nibble 0|1<<2 = 0x4) and
    # columns {2,3} in rows 2,3 (nibble 2|3<<2 = 0xE); columns likewise.
    assert c["meta_row"][0, 0] == 0x4444 and c["meta_row"][2, 0] == 0xEEEE
    assert c["meta_col"][0, 0] == 0x4444 and c["meta_col"][3, 0] == 0xEEEE
    assert c["vals_row"][0, :2].tolist() == [1, 2] and c["vals_row"][3, :2].tolist() == [15, 16]
    assert c["vals_col"][0, :2].tolist() == [1, 5] and c["vals_col"][2, :2].tolist() == [11, 15]


# ----------------------------------------------------------------------------
# GEMMs
def _spmm_loop(A, vals, meta, n_out, K):
    """float64 A[T,K] times the compressed [n_out, K] matrix, transposed, by explicit loops."""
    T = A.shape[0]
    out = np.zeros((T, n_out))
    for n in range(n_out):
        for g in range(K // 4):
            nib = (int(meta[n, g // 4]) >> (4 * (g % 4))) & 0xF
            for slot, k in ((0, 4 * g + (nib & 3)), (1, 4 * g + (nib >> 2))):
                w = float(vals[n, 2 * g + slot])
                out[:, n] += A[:, k].astype(np.float64) * w
    return out


def test_gemm_oracle_matches_explicit_loop():
    W = _w(19, 32, 48, "normal")
    idx = O.mask_search(W)
    c = O.compress(W, idx)
    rng = np.random.default_rng(20)
    X = rng.standard_normal((9, 48)).astype(np.float16)
    dY = rng.standard_normal((9, 32)).astype(np.float16)
    Y = O.spmm_fwd(X, c["vals_row"], c["meta_row"], 32, 48)
    dX = O.spmm_bwd_input(dY, c["vals_col"], c["meta_col"], 32, 48)
    np.testing.assert_allclose(Y, _spmm_loop(X, c["vals_row"], c["meta_row"], 32, 48), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dX, _spmm_loop(dY, c["vals_col"], c["meta_col"], 48, 32), rtol=1e-12, atol=1e-12)


def test_gemm_identity_special_cases():
    W = _w(21, 32, 16, "ints")
    idx = O.mask_search(W)
    c = O.compress(W, idx)
    pruned = np.where(O.idx_to_mask(idx), W, np.float16(0)).astype(np.float64)
    Y = O.spmm_fwd(np.eye(16, dtype=np.float16), c["vals_row"], c["meta_row"], 32, 16)
    assert (Y == pruned.T).all()                 # X = I gives Ws^T
    dX = O.spmm_bwd_input(np.eye(32, dtype=np.float16), c["vals_col"], c["meta_col"], 32, 16)
    assert (dX == pruned).all()                  # dY = I gives Ws


def test_gemm_error_metric():
    ref = np.array([[1.0, -2.0], [0.5, 4.0]])
    out = ref + np.array([[0.0, 0.04], [0.0, -0.02]])
    mr, ma = O.gemm_errors(out, ref)
    assert abs(mr - 0.01) < 1e-15 and abs(ma - 0.015) < 1e-15


# ----------------------------------------------------------------------------
# flip rate
def test_flip_count_pins():
    # identical masks do not flip; pattern 0 (1100 1100 0011 0011) and 89
    # (0011 0011 1100 1100) differ everywhere; patterns 0 and 1 (row 1 keeps
    # {0,2} instead of {0,1}, row 2 keeps {1,3} instead of {2,3}) differ in 4
    a = np.zeros((2, 3), np.uint8)
    assert O.flip_count(a, a) == 0
    b = a.copy()
    b[0, 0] = 89
    assert O.flip_count(a, b) == 16
    b[1, 2] = 1
    assert O.flip_count(a, b) == 20
    assert O.flip_rate(a, b) == 20 / 96


def test_flip_count_matches_dense_masks():
    rng = np.random.default_rng(30)
    W = (rng.standard_normal((64, 96)) * 0.02).astype(np.float16)
    W2 = (W.astype(np.float32) + rng.standard_normal(W.shape).astype(np.float32) * 1e-2).astype(np.float16)
    i1, i2 = O.mask_search(W), O.mask_search(W2)
    dense = int((O.idx_to_mask(i1) != O.idx_to_mask(i2)).sum())
    assert O.flip_count(i1, i2) == dense == O.flip_count(i2, i1)
    # flips within a block come in pairs (a row keeps exactly two entries)
    per_block = (O.idx_to_mask(i1) != O.idx_to_mask(i2)).reshape(16, 4, 24, 4).sum(axis=(1, 3))
    assert (per_block % 2 == 0).all() and per_block.max() <= 16
    # all 90 x 90 pattern pairs against explicit 4x4 comparisons
    masks = O.pattern_masks()
    p, q = np.meshgrid(np.arange(90), np.arange(90), indexing="ij")
    got = [O.flip_count(np.array([[x]], np.uint8), np.array([[y]], np.uint8)) for x, y in zip(p.ravel(), q.ravel())]
    want = [int((masks[x] != masks[y]).sum()) for x, y in zip(p.ravel(), q.ravel())]
    assert got == want


# ----------------------------------------------------------------------------
# weight gradient with masked decay
def test_weight_grad_explicit_loop():
    rng = np.random.default_rng(40)
    T, R, C = 5, 8, 12
    dY = rng.standard_normal((T, R)).astype(np.float16)
    X = rng.standard_normal((T, C)).astype(np.float16)
    W = rng.standard_normal((R, C)).astype(np.float16)
    idx = rng.integers(0, 90, size=(R // 4, C // 4)).astype(np.uint8)
    decay = 0.37
    masks = O.pattern_masks()
    want = np.zeros((R, C))
    for r in range(R):
        for c in range(C):
            s = 0.0
            for t in range(T):
                s += float(dY[t, r]) * float(X[t, c])
            kept = masks[idx[r // 4, c // 4], r % 4, c % 4]
            want[r, c] = s + (0.0 if kept else decay * float(W[r, c]))
    got = O.weight_grad(dY, X, W, idx, decay)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_weight_grad_special_cases():
    rng = np.random.default_rng(41)
    R, C = 16, 32
    W = rng.standard_normal((R, C)).astype(np.float16)
    idx = O.mask_search(W)
    # one-hot tokens: X = I picks the rows of dY, so dW = dY^T exactly
    dY = rng.standard_normal((C, R)).astype(np.float16)
    X = np.eye(C, dtype=np.float16)
    assert (O.weight_grad(dY, X, None, None, 0.0) == dY.astype(np.float64).T).all()
    # no tokens: only the decay term, which is zero on every kept entry and
    # decay * W on every pruned one, 8 of each 16 per block
    e = np.zeros((0, R), np.float16), np.zeros((0, C), np.float16)
    d = O.weight_grad(e[0], e[1], W, idx, 0.5)
    kept = O.idx_to_mask(idx).astype(bool)
    assert (d[kept] == 0).all()
    assert (d[~kept] == 0.5 * W.astype(np.float64)[~kept]).all()
    assert (~kept).reshape(R // 4, 4, C // 4, 4).sum(axis=(1, 3)).tolist() == [[8] * (C // 4)] * (R // 4)
    # linear in the decay factor, and decay 0 leaves the plain product
    dY2 = rng.standard_normal((7, R)).astype(np.float16)
    X2 = rng.standard_normal((7, C)).astype(np.float16)
    g0 = O.weight_grad(dY2, X2, W, idx, 0.0)
    g1 = O.weight_grad(dY2, X2, W, idx, 1.0)
    g3 = O.weight_grad(dY2, X2, W, idx, 3.0)
    assert np.allclose(g3 - g0, 3 * (g1 - g0), rtol=1e-12, atol=1e-12)
    assert (g0 == O.weight_grad(dY2, X2, None, None, 5.0)).all()


# ----------------------------------------------------------------------------
# GEGLU
def test_gelu_closed_forms():
    # GELU(0) = 0, GELU(x) - GELU(-x) = x, GELU'(0) = 1/2, GELU(x) -> x for
    # large x and -> 0 for very negative x; Phi(1) = 0.841344746068543 (table)
    x = np.array([0.0, 1.0, -1.0, 3.0, -3.0, 10.0, -10.0])
    g = O.gelu(x)
    assert g[0] == 0.0
    assert abs(g[1] - 0.841344746068543) < 1e-15
    assert np.allclose(g[1::2] - g[2::2], x[1::2], rtol=0, atol=1e-15)
    assert abs(g[5] - 10.0) < 1e-15 and abs(g[6]) < 1e-20
    assert O.gelu_grad(np.array([0.0]))[0] == 0.5
    # the negative tail keeps full relative accuracy: Phi(-6) = 9.865876450377e-10 (table)
    assert abs(O.gelu(np.array([-6.0]))[0] / -6.0 - 9.865876450377e-10) < 1e-12 * 9.865876450377e-10 * 100


def test_gelu_grad_matches_finite_differences():
    x = np.linspace(-6, 6, 241)
    h = 1e-6
    fd = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    assert np.allclose(O.gelu_grad(x), fd, rtol=0, atol=1e-8)


def test_geglu_layouts_and_backward():
    rng = np.random.default_rng(50)
    T, h = 3, 8
    v = rng.standard_normal((T, h))
    g = rng.standard_normal((T, h))
    # two halves (group = h): U = [v | g]
    U = np.concatenate([v, g], axis=1)
    assert np.allclose(O.geglu_fwd(U, h), v * O.gelu(g), rtol=0, atol=0)
    # group 2: v0 v1 g0 g1 v2 v3 g2 g3 ...
    U2 = np.concatenate([np.stack([v[:, 2 * b: 2 * b + 2], g[:, 2 * b: 2 * b + 2]], axis=1).reshape(T, 4)
                         for b in range(h // 2)], axis=1)
    assert (O.geglu_fwd(U2, 2) == O.geglu_fwd(U, h)).all()
    # the backward is the gradient of sum(dout * out) with respect to U
    dout = rng.standard_normal((T, h))
    dU = O.geglu_bwd(U2, dout, 2)
    eps = 1e-6
    num = np.zeros_like(U2)
    for t in range(T):
        for c in range(2 * h):
            up, dn = U2.copy(), U2.copy()
            up[t, c] += eps
            dn[t, c] -= eps
            num[t, c] = ((dout * O.geglu_fwd(up, 2)).sum() - (dout * O.geglu_fwd(dn, 2)).sum()) / (2 * eps)
    assert np.allclose(dU, num, rtol=0, atol=1e-7)


# ----------------------------------------------------------------------------
# MVUE
def _grid_stats(a, n=20000):
    """Mean and mean square of the estimate over u on a uniform grid of
    [0, 1) (the estimate is piecewise constant in u)."""
    mean = np.zeros(4)
    sq = np.zeros(4)
    hits = np.zeros(4)
    for j in range(n):
        u = np.float32((j + 0.5) / n)
        i, k, vi, vk = O.mvue_group(a, u)
        assert 0 <= i < k <= 3
        out = np.zeros(4)
        out[i], out[k] = float(vi), float(vk)
        mean += out
        sq += out * out
        hits[i] += 1
        hits[k] += 1
    return mean / n, sq / n, hits / n


def test_mvue_worked_examples():
    one = np.array([1, 1, 1, 1], np.float16)
    assert O.mvue_group(one, np.float32(0.25)) == (0, 2, 2.0, 2.0)      # C = 0.5, 1, 1.5
    assert O.mvue_group(one, np.float32(0.75)) == (1, 3, 2.0, 2.0)
    # u on a cumulative sum: the intervals are half-open, [C_(j-1), C_j)
    assert O.mvue_group(one, np.float32(0.5)) == (1, 3, 2.0, 2.0)       # u = C0, u + 1 = C2
    assert O.mvue_group(one, np.float32(0.0)) == (0, 2, 2.0, 2.0)       # u + 1 = C1
    dom = np.array([8, 1, 1, 0], np.float16)                          # p = 1 (capped), 1/2, 1/2, 0
    assert O.mvue_group(dom, np.float32(0.1)) == (0, 1, 8.0, 2.0)
    assert O.mvue_group(dom, np.float32(0.6)) == (0, 2, 8.0, 2.0)
    neg = np.array([-1, 3, 0, 0], np.float16)                         # p = 1/2, 3/2 -> capped: 1, 1
    i, k, vi, vk = O.mvue_group(neg, np.float32(0.3))
    assert (i, k, vi, vk) == (0, 1, -1.0, 3.0)
    # fewer than two non-zero entries: kept exactly
    assert O.mvue_group(np.array([0, 0, 3, 0], np.float16), np.float32(0.9)) == (0, 2, 0.0, 3.0)
    assert O.mvue_group(np.zeros(4, np.float16), np.float32(0.2)) == (0, 1, 0.0, 0.0)


def test_mvue_unbiased_with_minimum_variance():
    rng = np.random.default_rng(60)
    for trial in range(6):
        a = rng.standard_normal(4).astype(np.float16)
        if trial == 0:
            a[1] = np.float16(9.0)              # a capped entry
        if trial == 1:
            a[2] = np.float16(0.0)
        mean, sq, hits = _grid_stats(a)
        m = np.abs(a.astype(np.float64))
        p = 2 * m / m.sum()
        if p.max() > 1:
            kc = int(p.argmax())
            p = m / (m.sum() - m[kc])
            p[kc] = 1.0
        # unbiased, selected with probability p_i, variance a^2 (1/p - 1)
        assert np.allclose(mean, a.astype(np.float64), rtol=0, atol=2e-3 * np.abs(a).max())
        assert np.allclose(hits, p, atol=2e-4)
        var = sq - a.astype(np.float64) ** 2
        want = np.where(p > 0, a.astype(np.float64) ** 2 * (1 / np.where(p > 0, p, 1) - 1), 0)
        assert np.allclose(var, want, rtol=0, atol=5e-3 * (a.astype(np.float64) ** 2).max() + 1e-9)


def test_mvue_matches_exact_rational_definition():
    """Picks and kept values against the estimator's definition evaluated in
    exact rational arithmetic: p_i = 2|a_i|/S, the cap at 1 with the others
    rescaled by S - |a_k|, the cumulative sums, the intervals holding u and
    u + 1, and a_i / p_i.  Magnitudes span under 11 binades, so the fp32 sums
    are exact and so is the scale D (p_j = w_j / D).  No draw is skipped: the
    picks must be the definition's at u' = fl(u D) / D and u'' = fl(fl(u D) +
    D) / D, the fp32 reading for the uniform, and they must equal the
    definition's at u itself except within an fp32 rounding of a boundary.  A
    quarter of the draws put u on or next to a cumulative sum on purpose."""
    from fractions import Fraction as Fr
    f32 = np.float32
    rng = np.random.default_rng(62)
    checked = capped = moved = near = 0
    for _ in range(6000):
        mag = rng.uniform(0.25, 8.0, 4)
        mag[rng.random(4) < 0.1] *= 16.0            # some groups get a capped entry
        a = (rng.choice([-1.0, 1.0], 4) * mag).astype(np.float16)
        a[rng.random(4) < 0.15] = 0
        m = [abs(Fr(float(x))) for x in a]
        if sum(1 for x in m if x) < 2:
            continue
        S = sum(m)
        p = [2 * x / S for x in m]
        D = S / 2
        over = [j for j in range(4) if p[j] > 1]
        if over:
            kc = over[0]
            D = S - m[kc]
            p = [Fr(1) if j == kc else m[j] / D for j in range(4)]
        assert sum(p) == 2
        C = [p[0], p[0] + p[1], p[0] + p[1] + p[2]]
        u = f32(rng.random())
        if rng.random() < 0.25:
            # on a boundary: a cumulative sum (or one minus 1) rounded to fp32,
            # or its fp32 neighbour
            c = C[rng.integers(3)]
            t = float(c - 1) if c >= 1 else float(c)
            u = f32(t)
            if rng.random() < 0.5:
                u = np.nextafter(u, f32(rng.choice([-1.0, 2.0])), dtype=np.float32)
            if not 0 <= u < 1:
                continue
        uf = Fr(float(u))
        assert Fr(float(f32(float(D)))) == D                # D is exact in fp32
        uD = f32(u) * f32(float(D))
        u1 = Fr(float(uD)) / D
        u2 = Fr(float(f32(uD + f32(float(D))))) / D
        i = sum(c <= u1 for c in C)
        k = sum(c <= u2 for c in C)
        got = O.mvue_group(a, u)
        assert got[:2] == (i, k), (a, u)
        for j, v in ((i, got[2]), (k, got[3])):
            want = Fr(float(a[j])) / p[j] if p[j] else Fr(0)
            assert Fr(float(v)) == want, (a, u, j)
        # the definition at u itself: the same picks unless u is within an
        # fp32 rounding of a boundary
        i0, k0 = sum(c <= uf for c in C), sum(c <= uf + 1 for c in C)
        close = any(abs(c - uf) <= Fr(1, 2 ** 23) or abs(c - uf - 1) <= Fr(1, 2 ** 22) for c in C)
        near += close
        if (i0, k0) != (i, k):
            assert close, (a, u)
            moved += 1
        checked += 1
        capped += bool(over)
    assert checked > 4000 and capped > 300 and near > 500, (checked, capped, near)
    # the reading matters for some boundary draws, and only for those
    assert 0 < moved < near, (moved, near)
    print(f"{checked} draws, {capped} capped, {near} near a boundary, {moved} decided by the fp32 reading")


def test_mvue_last_interval_fallback():
    """fp32 rounding can put u in the last interval, which in exact arithmetic
    it never is (u < 1 <= C_2).  With magnitudes 1 - 2^-11, 1791 * 2^-22,
    1027 * 2^-24 and 1, the fp32 running sums are exact up to 1 - 2^-24, and
    adding the last 1 gives 2 - 2^-24, a tie that rounds to 2 (even).  So S = 2,
    D = 1, and u = 1 - 2^-24 satisfies W_2 <= u D: both u and u + 1 land in
    the last interval.  The picks are then the last two entries, which is also
    the exact answer: C_2 = (2 - 2^-23) / (2 - 2^-24) > u, and u + 1 > C_2."""
    from fractions import Fraction as Fr
    a = np.array([1 - 2.0 ** -11, 1791 * 2.0 ** -22, 1027 * 2.0 ** -24, 1.0], np.float16)
    u = np.float32(1 - 2.0 ** -24)
    assert [float(x) for x in a] == [1 - 2.0 ** -11, 1791 * 2.0 ** -22, 1027 * 2.0 ** -24, 1.0]
    w2 = np.float32(np.float32(np.float32(a[0]) + np.float32(a[1])) + np.float32(a[2]))
    assert w2 == np.float32(1 - 2.0 ** -24) and np.float32(w2 + np.float32(1)) == 2 and w2 <= u
    i, k, vi, vk = O.mvue_group(a, u)
    assert (i, k) == (2, 3)
    m = [Fr(float(x)) for x in a]
    S = sum(m)
    C = [2 * m[0] / S, 2 * (m[0] + m[1]) / S, 2 * (m[0] + m[1] + m[2]) / S]
    uf = Fr(float(u))
    assert sum(c <= uf for c in C) == 2 and sum(c <= uf + 1 for c in C) == 3
    # exact kept values are S / 2 = 1 - 2^-25; fp16 rounds both to 1
    assert np.float16(vi) == np.float16(float(S / 2)) == 1 and np.float16(vk) == np.float16(float(S / 2))


def test_mvue_matrix_form():
    rng = np.random.default_rng(61)
    M = rng.standard_normal((4, 32)).astype(np.float16)
    U = rng.random((4, 8), dtype=np.float32)
    f = O.mvue(M, U)
    for r in range(4):
        for g in range(8):
            i, k, vi, vk = O.mvue_group(M[r, 4 * g: 4 * g + 4], U[r, g])
            nib = (int(f["meta"][r, g // 4]) >> (4 * (g % 4))) & 0xF
            assert nib == (i | k << 2) and nib in (0x4, 0x8, 0xC, 0x9, 0xD, 0xE)
            assert f["vals"][r, 2 * g] == np.float16(vi) and f["vals"][r, 2 * g + 1] == np.float16(vk)
            # the estimate keeps the signs of the entries it keeps
            assert np.sign(float(vi)) in (0, np.sign(float(M[r, 4 * g + i])))
