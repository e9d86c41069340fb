"""CPU oracle for the transposable 2:4 FFN path.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  The HIP library never calls it, and it shares no
code, table or helper with the HIP path: the pattern list below is enumerated
here from its definition, independently of the GPU side's own table.

Source: "Accelerating Transformer Pre-training with 2:4 Sparsity" (Hu, Zhao,
Huang, Chen, Zhu; ICML 2024).  Cited as [HZ24 Alg.1] for Algorithm 1
(transposable mask search) on the reproducibility page, [HZ24 abstract] for
the abstract, and [HZ24 SW] for the page's "Software Dependencies" row, which
names the CUTLASS 2:4 sparse matrix multiplications and the Triton mask-search
and pruning kernels.

What the method computes, and the readings taken where the pages are silent:

1. Mask search [HZ24 Alg.1]: take |W|, correlate it with every mask pattern
   m using a 4x4 window at stride 4 and no padding, and return the argmax over
   patterns for each 4x4 block.
   * The pattern set m is every 4x4 0/1 matrix with exactly two ones in each
     row and each column.  These are the transposable 2:4 masks [HZ24
     abstract]: the block keeps 2 of 4 along rows and along columns.  There
     are 90 of them.
   * Pattern order (silent on the pages): each row keeps one of six column
     pairs, coded 0:{0,1} 1:{0,2} 2:{0,3} 3:{1,2} 4:{1,3} 5:{2,3}.  A pattern
     is a tuple (a, b, c, d) of codes for rows 0..3.  The list is every valid
     tuple in lexicographic order, a slowest.
   * The argmax is taken over the pattern axis (in the convolution's own
     output layout the axis the listing names would be a spatial one).
   * Score precision and order (silent): fp32, the kept magnitudes added one
     at a time in row-major order, starting from +0.
   * Tie-break (silent): the first maximum in pattern order (strict >).
   * R and C must be multiples of 4.  The stride-4 correlation without padding
     would drop a remainder, so the oracle refuses it instead.
2. Pruning and compression [HZ24 SW] (the format is not on the pages):
   * Row form: for row i and group g (columns 4g..4g+3) with kept in-group
     positions i0 < i1, ``vals_row[i, 2g:2g+2] = W[i, 4g+i0], W[i, 4g+i1]``
     (bit copies).  The nibble ``i0 | i1 << 2`` goes to bits 4*(g % 4) of the
     uint16 ``meta_row[i, g // 4]``.
   * Column form: the same applied to W transposed, so column j, group h (rows
     4h..4h+3) fills ``vals_col[j, 2h:2h+2]`` and ``meta_col[j, h // 4]``.
     Transposability [HZ24 abstract] makes every column group keep exactly 2.
   * Compression needs R and C to be multiples of 16, since a meta word holds
     four groups.
3. Sparse GEMMs [HZ24 abstract, SW]: ``Y = X Ws^T`` (forward) and
   ``dX = dY Ws`` (input gradient), with Ws the pruned weight.  The plain
   definition is the dense product with the decoded pruned matrix, computed
   here in float64.
4. Flip rate [HZ24 abstract] (no formula on the pages): the number of mask
   entries whose kept/pruned state differs between two consecutive masks,
   over the number of entries.
5. Weight gradient with masked decay [HZ24 abstract: the sparse-refined
   straight-through estimator, modified by applying the masked decay term on
   gradients; HZ24 SW: a masked-decay kernel].  No formula is on the pages.
   Reading: the gradient that reaches the dense weight is the straight-through
   product ``dY^T X`` (summed over tokens), and the masked decay term
   ``decay * (1 - M) * W`` (M the searched transposable mask, 1 where kept) is
   added to that gradient rather than applied to the weights.  Computed in
   float64; the library returns float32.
6. GEGLU [HZ24 abstract: accelerating gated activation functions; HZ24 SW:
   a GEGLU kernel].  The pages name the operation only.  Reading: the gated
   linear unit with a GELU gate, out = value * GELU(gate), GELU the exact
   x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), on the first linear's output U
   [T, 2h].  Column layout: blocks of G value columns followed by the G
   matching gate columns (G = h is the two-halves layout; a small G keeps each
   pair close together in memory).  The backward gives d value = dOut *
   GELU(gate) and d gate = dOut * value * GELU'(gate), GELU'(x) = Phi(x) + x
   phi(x).  Computed in float64.
7. MVUE [HZ24 SW: an MVUE kernel; only the name is on the pages].  Reading:
   the minimum-variance unbiased estimator that keeps 2 of every 4
   consecutive entries of a gradient row.  For a group a_0..a_3 the keep
   probabilities are p_i = 2|a_i| / S (S = sum |a_i|), which minimise the
   summed variance sum a_i^2 (1/p_i - 1) under sum p_i = 2; an entry with
   p_k > 1 is capped at 1 and the others get |a_j| / (S - |a_k|).  Exactly two
   entries are drawn by systematic sampling with one uniform u in [0, 1) per
   group (the cumulative sums C_0 .. C_2 of p; the picks are the interval
   holding u and the one holding u + 1), and a kept entry is a_i / p_i, which
   makes the estimate unbiased.  A group with fewer than two non-zero entries
   is kept as it is.  The output is the library's 2:4 row form.  Every
   decision is taken in fp32 in the order written in ``mvue_group``, so that
   an implementation with the same fp32 operations reproduces it bit for bit;
   that order compares cumulative masses with u times a scale instead of
   dividing (the same decisions in exact arithmetic), and a kept value is
   sign(a_i) times that scale, so no step divides.  The uniform enters only
   through two fp32 roundings, fl(u D) and fl(fl(u D) + D): within an fp32
   rounding of an interval boundary the picks are those of the definition at
   u' = fl(u D) / D (and u'' = fl(fl(u D) + D) / D for u + 1), not at u.
   That is the reading taken for such draws; elsewhere the two agree.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

# Column pairs a row may keep, coded 0..5 in lexicographic order.
ROW_PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def pattern_codes() -> list:
    """The transposable patterns as row-pair code tuples, in index order.

    Enumerates (a, b, c, d) over {0..5}^4 in lexicographic order and keeps a
    tuple when every column of the resulting 4x4 mask holds exactly two ones.
    """
    out = []
    for codes in itertools.product(range(6), repeat=4):
        colcount = [0, 0, 0, 0]
        for code in codes:
            for c in ROW_PAIRS[code]:
                colcount[c] += 1
        if colcount == [2, 2, 2, 2]:
            out.append(codes)
    return out


def pattern_masks() -> np.ndarray:
    """uint8 [90, 4, 4]: mask p has a one at (r, c) when pattern p keeps it."""
    codes = pattern_codes()
    m = np.zeros((len(codes), 4, 4), dtype=np.uint8)
    for p, tup in enumerate(codes):
        for r, code in enumerate(tup):
            for c in ROW_PAIRS[code]:
                m[p, r, c] = 1
    return m


def _check_shape(W: np.ndarray, mult: int) -> tuple:
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    R, C = W.shape
    if R <= 0 or C <= 0 or R % mult or C % mult:
        raise ValueError(f"W shape {W.shape} must be positive multiples of {mult}")
    return R, C


def _blocks(W: np.ndarray) -> np.ndarray:
    """[R/4, C/4, 4, 4] view of a [R, C] array, block (bi, bj) at [bi, bj]."""
    R, C = W.shape
    return W.reshape(R // 4, 4, C // 4, 4).transpose(0, 2, 1, 3)


def block_scores(W: np.ndarray) -> np.ndarray:
    """float32 [R/4, C/4, 90]: the per-block pattern scores of [HZ24 Alg.1].

    Step 1 takes |W| (fp16 -> fp32 is exact; the sign bit is cleared, so -0
    becomes +0).  Step 2 scores block (bi, bj) against pattern p by adding the
    kept magnitudes one at a time, in row-major order, in fp32.
    """
    W = np.asarray(W)
    if W.dtype != np.float16:
        raise TypeError("W must be float16")
    _check_shape(W, 4)
    A = _blocks(np.abs(W).astype(np.float32))
    masks = pattern_masks()
    out = np.empty(A.shape[:2] + (len(masks),), dtype=np.float32)
    for p, m in enumerate(masks):
        s = np.zeros(A.shape[:2], dtype=np.float32)
        for r in range(4):
            for c in range(4):
                if m[r, c]:
                    s = s + A[:, :, r, c]       # one fp32 add, round to nearest even
        out[:, :, p] = s
    return out


def mask_search(W: np.ndarray) -> np.ndarray:
    """uint8 [R/4, C/4] pattern index per 4x4 block [HZ24 Alg.1, step 3].

    The argmax keeps the first maximum in pattern order: a later pattern
    replaces the running best only when its score is strictly greater.
    """
    S = block_scores(W)
    best = np.zeros(S.shape[:2], dtype=np.uint8)
    best_s = S[:, :, 0].copy()
    for p in range(1, S.shape[2]):
        better = S[:, :, p] > best_s
        best = np.where(better, np.uint8(p), best)
        best_s = np.where(better, S[:, :, p], best_s)
    return best


def idx_to_mask(idx: np.ndarray) -> np.ndarray:
    """bool [R, C] mask of kept entries from the per-block pattern indices."""
    masks = pattern_masks().astype(bool)
    nbr, nbc = idx.shape
    return masks[idx].transpose(0, 2, 1, 3).reshape(4 * nbr, 4 * nbc)


def _compress_groups(W: np.ndarray, M: np.ndarray):
    """Compress along axis 1 in groups of 4: returns (vals [n, m/2], meta [n, m/16])."""
    n, m = W.shape
    G = m // 4
    Wg = W.reshape(n, G, 4)
    Mg = M.reshape(n, G, 4)
    if not (Mg.sum(axis=2) == 2).all():
        raise ValueError("every group of 4 must keep exactly 2")
    i0 = np.argmax(Mg, axis=2)                   # first kept position
    i1 = 3 - np.argmax(Mg[:, :, ::-1], axis=2)   # last kept position
    v0 = np.take_along_axis(Wg, i0[:, :, None], axis=2)[:, :, 0]
    v1 = np.take_along_axis(Wg, i1[:, :, None], axis=2)[:, :, 0]
    vals = np.stack([v0, v1], axis=2).reshape(n, m // 2)
    nib = (i0 | (i1 << 2)).astype(np.uint16).reshape(n, G // 4, 4)
    meta = nib[:, :, 0] | (nib[:, :, 1] << 4) | (nib[:, :, 2] << 8) | (nib[:, :, 3] << 12)
    return vals, meta.astype(np.uint16)


def compress(W: np.ndarray, idx: np.ndarray) -> dict:
    """Prune W with the searched masks and store both 2:4 forms.

    Returns ``vals_row`` fp16 [R, C/2], ``meta_row`` uint16 [R, C/16],
    ``vals_col`` fp16 [C, R/2] and ``meta_col`` uint16 [C, R/16].
    """
    W = np.asarray(W)
    if W.dtype != np.float16:
        raise TypeError("W must be float16")
    R, C = _check_shape(W, 16)
    if idx.shape != (R // 4, C // 4):
        raise ValueError("idx shape does not match W")
    if (idx >= 90).any():
        raise ValueError("pattern index out of range")
    M = idx_to_mask(idx)
    vals_row, meta_row = _compress_groups(W, M)
    vals_col, meta_col = _compress_groups(np.ascontiguousarray(W.T), np.ascontiguousarray(M.T))
    return {"vals_row": vals_row, "meta_row": meta_row,
            "vals_col": vals_col, "meta_col": meta_col}


def _decode_groups(vals: np.ndarray, meta: np.ndarray, n: int, m: int) -> np.ndarray:
    """Inverse of ``_compress_groups``: fp16 [n, m], +0 where nothing is kept."""
    out = np.zeros((n, m // 4, 4), dtype=np.float16)
    v = vals.reshape(n, m // 4, 2)
    for g in range(m // 4):
        nib = (meta[:, g // 4].astype(np.int64) >> (4 * (g % 4))) & 0xF
        i0, i1 = nib & 3, nib >> 2
        rows = np.arange(n)
        out[rows, g, i0] = v[:, g, 0]
        out[rows, g, i1] = v[:, g, 1]
    return out.reshape(n, m)


def decode_row_form(vals_row, meta_row, R: int, C: int) -> np.ndarray:
    """Dense fp16 [R, C] pruned weight from the row form."""
    return _decode_groups(vals_row, meta_row, R, C)


def decode_col_form(vals_col, meta_col, R: int, C: int) -> np.ndarray:
    """Dense fp16 [R, C] pruned weight from the column form."""
    return _decode_groups(vals_col, meta_col, C, R).T


def spmm_fwd(X: np.ndarray, vals_row, meta_row, R: int, C: int) -> np.ndarray:
    """float64 [T, R]: Y = X Ws^T with Ws decoded from the row form."""
    Ws = decode_row_form(vals_row, meta_row, R, C).astype(np.float64)
    return np.asarray(X, dtype=np.float64) @ Ws.T


def spmm_bwd_input(dY: np.ndarray, vals_col, meta_col, R: int, C: int) -> np.ndarray:
    """float64 [T, C]: dX = dY Ws with Ws decoded from the column form."""
    Ws = decode_col_form(vals_col, meta_col, R, C).astype(np.float64)
    return np.asarray(dY, dtype=np.float64) @ Ws


def flip_count(idx_prev: np.ndarray, idx_new: np.ndarray) -> int:
    """Number of mask entries that differ between two searched masks.

    [HZ24 abstract] defines a "flip rate" to monitor the stability of 2:4
    training but prints no formula.  Reading: the entries whose kept/pruned
    state changed between two consecutive masks, counted over the whole
    matrix; ``flip_rate`` divides by the number of entries.
    """
    if idx_prev.shape != idx_new.shape:
        raise ValueError("mask shapes differ")
    masks = pattern_masks().astype(np.int64)
    diff = masks[idx_prev.astype(np.int64)] != masks[idx_new.astype(np.int64)]
    return int(diff.sum())


def flip_rate(idx_prev: np.ndarray, idx_new: np.ndarray) -> float:
    """flip_count divided by the number of matrix entries (16 per block)."""
    n = 16 * idx_new.size
    return flip_count(idx_prev, idx_new) / n if n else 0.0


def weight_grad(dY: np.ndarray, X: np.ndarray, W: np.ndarray | None, idx: np.ndarray | None,
                decay: float) -> np.ndarray:
    """``dW = dY^T X + decay * (1 - M) * W`` in float64 (item 5 above).

    dY [T, R] and X [T, C] are the output gradient and the input of the
    linear layer; W [R, C] its dense weight and idx [R/4, C/4] the searched
    masks.  With W or idx None the decay term is left out.
    """
    dW = dY.astype(np.float64).T @ X.astype(np.float64)
    if W is not None and idx is not None:
        pruned = 1.0 - idx_to_mask(idx).astype(np.float64)
        dW = dW + float(decay) * pruned * W.astype(np.float64)
    return dW


def _geglu_split(U: np.ndarray, group: int):
    """Value and gate columns of U [T, 2h] laid out in blocks of `group`."""
    T, two_h = U.shape
    if two_h % (2 * group) != 0:
        raise ValueError("2h must be a multiple of 2 * group")
    blocks = U.astype(np.float64).reshape(T, two_h // (2 * group), 2, group)
    return blocks[:, :, 0, :].reshape(T, -1), blocks[:, :, 1, :].reshape(T, -1)


_erfc = np.vectorize(math.erfc, otypes=[np.float64])


def _phi_cdf(x: np.ndarray) -> np.ndarray:
    """Phi(x) = erfc(-x / sqrt 2) / 2, the form that keeps its relative
    accuracy in the negative tail (1 + erf(x / sqrt 2) cancels there)."""
    return 0.5 * _erfc(-x / math.sqrt(2.0))


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x * Phi(x), in float64."""
    return x * _phi_cdf(x)


def gelu_grad(x: np.ndarray) -> np.ndarray:
    """d GELU / dx = Phi(x) + x * phi(x)."""
    return _phi_cdf(x) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def geglu_fwd(U: np.ndarray, group: int) -> np.ndarray:
    """out [T, h] = value * GELU(gate) (item 6 above), float64."""
    v, g = _geglu_split(U, group)
    return v * gelu(g)


def geglu_bwd(U: np.ndarray, dout: np.ndarray, group: int) -> np.ndarray:
    """dU [T, 2h] in U's layout: d value = dout * GELU(gate), d gate =
    dout * value * GELU'(gate) (item 6 above), float64."""
    v, g = _geglu_split(U, group)
    d = dout.astype(np.float64)
    dv, dg = d * gelu(g), d * v * gelu_grad(g)
    T, h = dv.shape
    out = np.empty((T, h // group, 2, group))
    out[:, :, 0, :] = dv.reshape(T, -1, group)
    out[:, :, 1, :] = dg.reshape(T, -1, group)
    return out.reshape(T, 2 * h)


def mvue_group(a: np.ndarray, u: np.float32) -> tuple:
    """One group of item 7: a = 4 fp16 values, u = fp32 uniform in [0, 1).

    Returns (i, k, value_i, value_k) with i < k, values as fp32.  All
    arithmetic is fp32 (numpy float32 scalars round every operation).

    The probabilities are carried as masses w_j over a common scale D, with
    p_j = w_j / D and sum p_j = 2 (so sum w_j = 2 D):
      uncapped  w_j = |a_j|, D = S / 2;
      capped k  w_j = |a_j| for j != k, w_k = D = S - |a_k| (so p_k = 1).
    A cumulative sum C_j = W_j / D (W_j = w_0 + .. + w_j) is compared with u
    as W_j <= u D, and with u + 1 as W_j <= u D + D.  A kept entry's value
    a_j / p_j is then a_j itself for the capped entry and sign(a_j) D for
    any other entry with a_j != 0.  In exact arithmetic this is the
    definition; in fp32 it has no division, and every sum of fp16
    magnitudes in it is exact unless they span more than 11 binades.
    """
    f = np.float32
    m = [f(abs(f(x))) for x in a]
    nz = [i for i in range(4) if m[i] != 0]
    if len(nz) < 2:
        # nothing to sample: keep the non-zero entry (if any) and the lowest
        # other index, both exactly
        i = nz[0] if nz else 0
        k = 1 if i == 0 else 0
        i, k = min(i, k), max(i, k)
        return i, k, f(a[i]), f(a[k])
    S = f(f(f(m[0] + m[1]) + m[2]) + m[3])
    # p_k > 1  <=>  2 |a_k| > S; at most one entry can satisfy it
    over = [i for i in range(4) if f(2) * m[i] > S]
    kc = over[0] if over else -1
    if kc >= 0:
        D = f(0)
        for j in range(4):
            if j != kc:
                D = f(D + m[j])
        w = [D if j == kc else m[j] for j in range(4)]
    else:
        D = f(S * f(0.5))
        w = m
    W0 = w[0]
    W1 = f(W0 + w[1])
    W2 = f(W1 + w[2])
    uD = f(f(u) * D)
    uD1 = f(uD + D)
    i = int(W0 <= uD) + int(W1 <= uD) + int(W2 <= uD)
    k = int(W0 <= uD1) + int(W1 <= uD1) + int(W2 <= uD1)
    if k == i:
        # Only possible in the last interval.  Every mass is at most D, and
        # fp32 rounding is monotone, so W_i = fl(W_(i-1) + w_i) <= fl(uD + D)
        # whenever W_(i-1) <= uD: u + 1 always lies past u's interval when
        # that is not the last.  u's interval is the last only by rounding (in
        # exact arithmetic u < 1 <= C_2): W_2 <= fl(u D) needs a sum that rounds
        # up, outside the 11-binade range where the sums are exact.  The picks
        # are then the last two entries.
        assert i == 3, "u and u + 1 share an interval before the last"
        i, k = 2, 3

    def val(j):
        if j == kc:
            return f(a[j])
        return f(np.copysign(D, f(a[j]))) if m[j] != 0 else f(0)

    return i, k, val(i), val(k)


def mvue(M: np.ndarray, U: np.ndarray) -> dict:
    """Item 7 over a matrix: M fp16 [rows, cols] (cols a multiple of 16),
    U fp32 [rows, cols/4].  Returns the row form {"vals": fp16 [rows,
    cols/2], "meta": uint16 [rows, cols/16]}."""
    rows, cols = M.shape
    if cols % 16 != 0 or U.shape != (rows, cols // 4):
        raise ValueError("cols must be a multiple of 16 and U [rows, cols/4]")
    vals = np.zeros((rows, cols // 2), np.float16)
    meta = np.zeros((rows, cols // 16), np.uint16)
    for r in range(rows):
        for g in range(cols // 4):
            i, k, vi, vk = mvue_group(M[r, 4 * g: 4 * g + 4], U[r, g])
            vals[r, 2 * g] = np.float16(vi)
            vals[r, 2 * g + 1] = np.float16(vk)
            meta[r, g // 4] |= np.uint16((i | (k << 2)) << (4 * (g % 4)))
    return {"vals": vals, "meta": meta}


def gemm_errors(out: np.ndarray, ref: np.ndarray) -> tuple:
    """(normwise max relative error, mean absolute error) of ``out`` vs ``ref``.

    The relative error is max|out - ref| / max|ref|: an elementwise relative
    error is unbounded where ref is near zero, for any finite-precision result.
    """
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    diff = np.abs(o - r)
    denom = np.abs(r).max() if r.size else 0.0
    max_rel = float(diff.max() / denom) if r.size and denom > 0 else float(diff.max() if r.size else 0.0)
    mean_abs = float(diff.mean()) if r.size else 0.0
    return max_rel, mean_abs
