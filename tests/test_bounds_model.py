"""Host model of the kernels' address arithmetic (CPU only, no kernel runs).

For every shape the GPU tests and the benchmark use, the index formulas of
the HIP kernels are replayed here in numpy, and the test checks that:

* every tile of a launch is visited exactly once (the workgroup -> tile maps,
  the tail split and the grouped launch's per-XCD queues);
* every output element is written exactly once, and only inside its buffer
  (the epilogues' lane -> element maps with their bounds checks);
* every direct-load offset fits the 32-bit signed arithmetic the kernels form
  it in, and each buffer descriptor's base and byte range lie inside the
  operand it reads (rows past the end then read as zero, by design);
* the compressed forms' addresses (the search's stores, the GEMMs' loads,
  MVUE's stores) are where the header's blocked order puts each element,
  taken from tests/forms_layout.py's construction of that order.

The formulas are transcribed from the sources named in each function
(structured_sparse_transformer_amd/csrc); a change to a kernel's indexing has
to be mirrored here.  The device is modelled with 256 CUs.
"""
import numpy as np
import pytest

from structured_sparse_transformer_amd import workloads as WL

from forms_layout import META_BLOCK, VALS_BLOCK, blocked_positions

CUS = 256
I32 = 2 ** 31
U32 = 2 ** 32


def cdiv(a, b):
    return -(-a // b)


# ----------------------------------------------------------------------------
# workgroup -> tile maps

def xcd_run_map(ntiles, grid):
    """blockIdx -> linear tile of the single launches (sp24_spmm.hip,
    sp24_dw.hip): XCD b % 8 walks a contiguous run of the tile order."""
    per_xcd = cdiv(ntiles, 8)
    b = np.arange(grid)
    lin = (b % 8) * per_xcd + b // 8
    return lin[lin < ntiles]


def group_order(lin, tiles_m, tiles_n, group_m=8):
    """Linear position -> (tm, tn): groups of 8 row tiles, column tiles within
    a group, rows fastest."""
    group = lin // (group_m * tiles_n)
    gm0 = group * group_m
    gsize = np.minimum(group_m, tiles_m - gm0)
    in_group = lin - group * group_m * tiles_n
    return gm0 + in_group % gsize, in_group // gsize


def check_tile_map(tiles_m, tiles_n):
    grid = cdiv(tiles_m * tiles_n, 8) * 8
    tm, tn = group_order(xcd_run_map(tiles_m * tiles_n, grid), tiles_m, tiles_n)
    seen = np.zeros((tiles_m, tiles_n), np.int64)
    np.add.at(seen, (tm, tn), 1)
    assert (seen == 1).all(), "a tile is missed or visited twice"
    return tm, tn


# ----------------------------------------------------------------------------
# sparse GEMM (sp24_spmm.hip)

def fast_path(T, N, K):
    return K % 64 == 0 and K > 0 and K * 512 < I32 and T * K * 2 < I32 and N * K < I32 and T * N * 2 < 2 ** 40


def tail_tiles(T, w):
    return 2 * cdiv(T, 128) if w > 128 else cdiv(T, 64)


def split_features(T, N):
    tiles_n, tiles_m = cdiv(T, 256), cdiv(N, 256)
    if tiles_m < 2 or (tiles_m * tiles_n) % CUS == 0 or ((tiles_m - 1) * tiles_n) % CUS != 0:
        return 0
    n1 = (tiles_m - 1) * 256
    return n1 if tail_tiles(T, N - n1) <= CUS else 0


def fast_launches(T, N, K):
    """launch_spmm_nt's fast-path launches: (BM, BN, WM, WN, first feature, features)."""
    n1 = split_features(T, N)
    if n1 == 0:
        return [(256, 256, 128, 64, 0, N)]
    tail = (128, 128, 128, 32) if N - n1 > 128 else (256, 64, 128, 32)
    return [(256, 256, 128, 64, 0, n1), tail + (n1, N - n1)]


def swz_s(r):
    return ((r >> 1) ^ (r >> 2)) & 3


def swz_b(r):
    return (r & 7) ^ ((r >> 3) & 1)


def fast_tile_writes(BM, BN, WM, WN):
    """(token, feature) of every 16-byte store of spmm_fast_tile's epilogue,
    relative to the tile: lane t of wave (wm, wn) writes row t/16 + 4 it,
    chunk t % 16 (8 features), it < WN*16/64."""
    waves = (BM // WM) * (BN // WN)
    rows, cols = [], []
    for wave in range(waves):
        wm, wn = wave % (BM // WM), wave // (BM // WM)
        for it in range(WN * 16 // 64):
            lane = np.arange(64)
            t, c = it * 4 + lane // 16, lane % 16
            rows.append(wn * WN + t)
            cols.append(wm * WM + c * 8)
    return np.concatenate(rows), np.concatenate(cols)


def check_fast_tile_pattern(BM, BN, WM, WN):
    n, m = fast_tile_writes(BM, BN, WM, WN)
    assert WM == 128 and (m % 8 == 0).all()
    cover = np.zeros((BN, BM // 8), np.int64)
    np.add.at(cover, (n, m // 8), 1)
    assert (cover == 1).all(), f"the {BM}x{BN} epilogue does not write its tile exactly once"
    return n, m


def fast_s_meta_offsets(BM, BN, WM, WN, N, K, m0):
    """spmm_fast_tile's per-lane byte offsets of stage 0 for S and meta and
    each load's stage stride, with the (row, 16-byte chunk) of S and (row,
    dword) of meta each lane fetches: lists over (wave, load) of (row, chunk,
    offset, stride)."""
    waves = (BM // WM) * (BN // WN)
    s_loads, m_loads = BM * 64 // 1024 // waves, BM * 8 // 256 // waves
    band_s, band_m = 64 * K, 8 * K

    def band_rows(band):
        return max(0, min(64, N - m0 - 64 * band))

    lane = np.arange(64)
    s_out, m_out = [], []
    for wave in range(waves):
        for i in range(s_loads):
            r = 16 * (wave * s_loads + i) + lane // 4
            chunk = (lane % 4) ^ swz_s(r)
            st = band_rows((wave * s_loads + i) // 4) * 64
            assert (r // 64 == (wave * s_loads + i) // 4).all()
            s_out.append((r, chunk, (r // 64) * band_s + (r % 64) * 64 + chunk * 16, st))
        for i in range(m_loads):
            r = 32 * (wave * m_loads + i) + lane // 2
            st = band_rows((wave * m_loads + i) // 2) * 8
            assert (r // 64 == (wave * m_loads + i) // 2).all()
            m_out.append((r, lane % 2, (r // 64) * band_m + (r % 64) * 8 + (lane % 2) * 4, st))
    return s_out, m_out


def check_fast_loads(BM, BN, WM, WN, T, N, K, m0, n0):
    """Direct-load offsets of one tile (int32 arithmetic) and its descriptors."""
    waves = (BM // WM) * (BN // WN)
    nk = K // 64
    b_loads = BN * 128 // 1024 // waves
    lane = np.arange(64)
    s_out, m_out = fast_s_meta_offsets(BM, BN, WM, WN, N, K, m0)
    worst = max(max(int(off.max()) + (nk - 1) * st for _, _, off, st in s_out),
                max(int(off.max()) + (nk - 1) * st for _, _, off, st in m_out))
    for wave in range(waves):
        for i in range(b_loads):
            r = 8 * (wave * b_loads + i) + lane // 8
            off = r * K * 2 + ((lane % 8) ^ swz_b(r)) * 16
            worst = max(worst, int(off.max()) + (nk - 1) * 128)
    assert worst + 16 <= I32, "a direct-load offset overflows 32-bit arithmetic"
    # descriptors: from this tile's first row to the operand's end (S: N x K/2
    # halves, meta: N x K/16 words, activations: T x K halves)
    for base, rng, total in ((m0 * K, (N - m0) * K, N * K), (n0 * K * 2, (T - n0) * K * 2, T * K * 2),
                             (m0 * K // 8, (N - m0) * K // 8, N * K // 8)):
        assert 0 <= base and base + rng == total and 0 < rng < U32


def check_fast_form_loads(BM, BN, WM, WN, N_all, f0, N, K, m0):
    """Each S and meta load of a tile at feature row m0 of a launch over rows
    f0 .. f0+N of an N_all-row operand (a tail launch passes vals and meta
    advanced by f0 rows) fetches, at every stage, the bytes the operand's
    blocked order holds for its (row, chunk); rows past N start beyond the
    descriptor's range (they load zeros)."""
    nk = K // 64
    ps, pm = blocked_positions(N_all, K // 2, VALS_BLOCK), blocked_positions(N_all, K // 16, META_BLOCK)
    s_out, m_out = fast_s_meta_offsets(BM, BN, WM, WN, N, K, m0)
    for kt in sorted({0, nk // 2, nk - 1}):
        for r, chunk, off, st in s_out:
            inside = m0 + r < N
            want = ps[f0 + m0 + r[inside], 32 * kt + 8 * chunk[inside]] * 2
            at = off + kt * st
            assert (f0 * K + m0 * K + at[inside] == want).all(), "S load off its block"
            # rows past N: whole 16-byte reads inside the operand, or past its end
            past = at[~inside]
            assert ((past + 16 <= (N - m0) * K) | (past >= (N - m0) * K)).all()
        for r, dw, off, st in m_out:
            inside = m0 + r < N
            want = pm[f0 + m0 + r[inside], 4 * kt + 2 * dw[inside]] * 2
            at = off + kt * st
            assert ((f0 + m0) * K // 8 + at[inside] == want).all(), "meta load off its block"
            past = at[~inside]
            assert ((past + 4 <= (N - m0) * K // 8) | (past >= (N - m0) * K // 8)).all()


def check_spmm(T, N, K):
    """Every output element of out[T][N] = A S^T written once, in bounds."""
    if T == 0 or N == 0:
        return
    cover = np.zeros((T, N // 8), np.int8)
    if fast_path(T, N, K):
        for BM, BN, WM, WN, f0, nf in fast_launches(T, N, K):
            tiles_m, tiles_n = cdiv(nf, BM), cdiv(T, BN)
            tm, tn = check_tile_map(tiles_m, tiles_n)
            n_rel, m_rel = check_fast_tile_pattern(BM, BN, WM, WN)
            for a in range(tiles_m):
                check_fast_form_loads(BM, BN, WM, WN, N, f0, nf, K, a * BM)
            for a, b in zip(tm, tn):
                m0, n0 = a * BM, b * BN
                check_fast_loads(BM, BN, WM, WN, T, nf, K, m0, n0)
                n, m = n0 + n_rel, m0 + m_rel
                ok = (n < T) & (m < nf)             # the epilogue's bounds check
                assert (m[ok] + 8 <= nf).all()
                np.add.at(cover, (n[ok], (f0 + m[ok]) // 8), 1)
    else:
        # spmm_nt_kernel (256 x 128 tiles, waves of 128 x 64): lane (l32, g)
        # of wave (wm, wn) writes 4 features 8 i4 + 4 g of each 32-feature
        # block mt, token l32 of block nt; rows are clamped on load
        BM, BN, WM, WN = 256, 128, 128, 64
        tiles_m, tiles_n = cdiv(N, BM), cdiv(T, BN)
        tm, tn = check_tile_map(tiles_m, tiles_n)
        lane = np.arange(64)
        l32, g = lane & 31, lane >> 5
        rel_n, rel_m = [], []
        for wave in range(4):
            wm, wn = wave % 2, wave // 2
            for mt in range(WM // 32):
                for nt in range(WN // 32):
                    for i4 in range(4):
                        rel_n.append(wn * WN + nt * 32 + l32)
                        rel_m.append(wm * WM + mt * 32 + 8 * i4 + 4 * g)
        rel_n, rel_m = np.concatenate(rel_n), np.concatenate(rel_m)
        quad = np.zeros((BN, BM // 4), np.int64)
        np.add.at(quad, (rel_n, rel_m // 4), 1)
        assert (quad == 1).all()
        cover4 = np.zeros((T, N // 4), np.int8)
        for a, b in zip(tm, tn):
            n, m = b * BN + rel_n, a * BM + rel_m
            ok = (n < T) & (m < N)
            assert (m[ok] + 4 <= N).all()
            np.add.at(cover4, (n[ok], m[ok] // 4), 1)
        assert (cover4 == 1).all()
        return
    assert (cover == 1).all(), "an output element is written twice or not at all"


def group_queues(jobs):
    """The grouped launch's queues (launch_spmm_group, spmm_group_kernel):
    jobs sorted by K, longest first; run x of each job's tile order per XCD."""
    order = sorted(range(len(jobs)), key=lambda j: -jobs[j][2])
    tiles = []
    for x in range(8):
        for q in order:
            T, N, K = jobs[q]
            tiles_m, tiles_n = cdiv(N, 256), cdiv(T, 256)
            nt = tiles_m * tiles_n
            lo, hi = x * nt // 8, (x + 1) * nt // 8
            tm, tn = group_order(np.arange(lo, hi), tiles_m, tiles_n)
            tiles += [(q, int(a), int(b)) for a, b in zip(tm, tn)]
    return tiles


# ----------------------------------------------------------------------------
# weight gradient (sp24_dw.hip)

# (BM, BN, WM, WN, relative speed, may split the tokens)
DW_SHAPES = [(256, 256, 128, 128, 1.0, False), (256, 320, 128, 160, 0.97, True), (320, 256, 160, 128, 0.97, True),
             (256, 160, 64, 160, 0.9, False), (160, 256, 160, 64, 0.9, False), (128, 128, 64, 64, 0.75, False)]
DW_FLAG_TILES = 256


def dw_shape(T, R, C):
    """launch_weight_grad's choice: (BM, BN, WM, WN, split)."""
    best, best_t, best_split = None, 0.0, False
    stages = cdiv(T, 32)
    for k, (bm, bn, wm, wn, speed, splittable) in enumerate(DW_SHAPES):
        tiles = cdiv(R, bm) * cdiv(C, bn)
        area = bm * bn / speed
        t = cdiv(tiles, CUS) * area
        split = False
        whole = R % bm == 0 and C % bn == 0
        if (splittable and whole and 2 * tiles <= CUS and 8 * tiles >= 3 * CUS and tiles <= DW_FLAG_TILES
                and stages >= 2 and area / 2 < t):
            t, split = area / 2, True
        if best is None or t < best_t:
            best, best_t, best_split = k, t, split
    return DW_SHAPES[best][:4] + (best_split,)


def dw_roles(tiles_m, tiles_n, split):
    """weight_grad_kernel's workgroup -> (tile, role) map: role 0 whole, 1 the
    first half of the tokens (consumer), 2 the second half (producer)."""
    ntiles = tiles_m * tiles_n
    per_run = cdiv(ntiles, 4 if split else 8)
    out = []
    for b in range(8 * per_run):
        xcd, in_xcd = b % 8, b // 8
        role = 0 if not split else (2 if xcd < 4 else 1)
        lin = (xcd % 4 if split else xcd) * per_run + in_xcd
        if in_xcd < per_run and lin < ntiles:
            out.append((b, lin, role))
    return out


def dw_tile(lin, tiles_m, tiles_n, split):
    """weight_grad_kernel's tile of run position lin: groups of 8 row tiles
    (whole), or across the grid's shorter side first (split)."""
    if not split:
        lm, ln = group_order(np.array([lin]), tiles_m, tiles_n)
        return int(lm[0]), int(ln[0])
    return (lin // tiles_n, lin % tiles_n) if tiles_n <= tiles_m else (lin % tiles_m, lin // tiles_m)


def dw_l2_fill_bytes(T, R, C, bm, bn, split):
    """Bytes of dY and X that the XCDs' L2s fetch, each XCD its tiles' operand
    strips once over its token range (the model behind the split's tile map)."""
    tiles_m, tiles_n = cdiv(R, bm), cdiv(C, bn)
    rows, cols = [set() for _ in range(8)], [set() for _ in range(8)]
    for b, lin, _ in dw_roles(tiles_m, tiles_n, split):
        a, c = dw_tile(lin, tiles_m, tiles_n, split)
        rows[b % 8].add(a)
        cols[b % 8].add(c)
    tokens = T // 2 if split else T
    return sum((len(r) * bm + len(c) * bn) * tokens * 2 for r, c in zip(rows, cols))


def check_weight_grad(T, R, C):
    BM, BN, WM, WN, split = dw_shape(T, R, C)
    tiles_m, tiles_n = cdiv(R, BM), cdiv(C, BN)
    if not split:
        check_tile_map(tiles_m, tiles_n)
    roles = dw_roles(tiles_m, tiles_n, split)
    # every tile once (whole), or once as producer (XCDs 0-3) and once as
    # consumer (XCDs 4-7), the producer with the lower workgroup id
    per_tile = {}
    for b, lin, role in roles:
        per_tile.setdefault(lin, []).append((role, b))
    assert sorted(per_tile) == list(range(tiles_m * tiles_n))
    for lin, rs in per_tile.items():
        if split:
            (r1, b1), (r2, b2) = sorted(rs)
            assert (r1, r2) == (1, 2) and b2 < b1 and b2 % 8 < 4 and b1 % 8 == b2 % 8 + 4
        else:
            assert [r for r, _ in rs] == [0]
    waves = (BM // WM) * (BN // WN)
    lane = np.arange(64)
    l32, g = lane & 31, lane >> 5
    rel_r, rel_c = [], []
    for wave in range(waves):
        wm, wn = wave % (BM // WM), wave // (BM // WM)
        for mt in range(WM // 32):
            for nt in range(WN // 32):
                for i4 in range(4):
                    rel_c.append(wn * WN + nt * 32 + l32)
                    rel_r.append(wm * WM + mt * 32 + 8 * i4 + 4 * g)
    rel_r, rel_c = np.concatenate(rel_r), np.concatenate(rel_c)
    quad = np.zeros((BM // 4, BN), np.int64)
    np.add.at(quad, (rel_r // 4, rel_c), 1)
    assert (quad == 1).all(), "the weight-gradient epilogue does not cover its tile once"
    cover = np.zeros((R // 4, C), np.int8)
    nk_all = cdiv(T, 32)
    tiles_seen = np.zeros((tiles_m, tiles_n), np.int64)
    for lin in range(tiles_m * tiles_n):
        a, b = dw_tile(lin, tiles_m, tiles_n, split)   # the kernel's lin -> tile
        tiles_seen[a, b] += 1
        m0, n0 = a * BM, b * BN
        r4, c = m0 + rel_r, n0 + rel_c
        ok = (r4 < R) & (c < C)
        assert (r4[ok] + 4 <= R).all()
        np.add.at(cover, (r4[ok] // 4, c[ok]), 1)   # the final store (whole or consumer)
        # direct loads of each role: 32 token rows per stage from token t0 on,
        # offsets row*R*2 + slot*16 + kt*32*R*2 in 32-bit arithmetic
        ranges = [(0, nk_all)] if not split else [(0, nk_all // 2), (nk_all // 2, nk_all - nk_all // 2)]
        assert sum(n for _, n in ranges) == nk_all
        for k_lo, nk in ranges:
            if T == 0 or nk == 0:
                continue
            t0 = k_lo * 32
            worst_a = 31 * R * 2 + (BM // 8 - 1) * 16 + (nk - 1) * 32 * R * 2
            worst_b = 31 * C * 2 + (BN // 8 - 1) * 16 + (nk - 1) * 32 * C * 2
            assert max(worst_a, worst_b) + 16 <= I32
            for base, rng, total in (((t0 * R + m0) * 2, ((T - t0) * R - m0) * 2, T * R * 2),
                                     ((t0 * C + n0) * 2, ((T - t0) * C - n0) * 2, T * C * 2)):
                assert base + rng == total and 0 < rng < U32
    assert (cover == 1).all() and (tiles_seen == 1).all()
    if split:
        assert tiles_m * tiles_n <= DW_FLAG_TILES


# ----------------------------------------------------------------------------
# search + compression (sp24_search.hip), 128 x 128 tiles, 256 threads

TILE, THREADS, TILES_PER_WG = 128, 256, 1


def form_off(r, c, n, m, b):
    """sp24_internal.hpp's form_off: the offset of (r, c) of an n x m form
    matrix in blocked order (bands of 64 rows, column blocks of width b)."""
    r0, c0 = r & ~63, c & ~(b - 1)
    h, w = np.minimum(64, n - r0), np.minimum(b, m - c0)
    return r0 * m + c0 * h + (r - r0) * w + (c - c0)


def full_tile_form_offsets(n, m, b, r0, c0s, r, g4, kk):
    """write_full_tile's offset of row r0 + r + 32 kk, segment g4 of a form
    matrix n x m (vals: segments of 8 halves, b = 32, c0s = c0 / 2; meta:
    words, b = 4, c0s = c0 / 16)."""
    seg = 8 if b == VALS_BLOCK else 1
    inner = (g4 // 4) * 64 * b + r * b + seg * (g4 % 4)
    return r0 * m + c0s * 64 + inner + (kk // 2) * 64 * m + (kk % 2) * 32 * b


def check_search_compress(shapes):
    """One batched launch over `shapes`: tiles map onto jobs once, and the
    index, both values and both meta outputs of every job are written once."""
    begin, total = [], 0
    for R, C in shapes:
        begin.append(total)
        total += cdiv(R, TILE) * cdiv(C, TILE)
    groups = cdiv(total, TILES_PER_WG)
    grid = cdiv(groups, 8) * 8
    per_xcd = cdiv(groups, 8)
    b = np.arange(grid)
    grp = (b % 8) * per_xcd + b // 8
    ts = [int(gp) * TILES_PER_WG + k for gp in grp[grp < groups] for k in range(TILES_PER_WG)
          if int(gp) * TILES_PER_WG + k < total]
    assert sorted(ts) == list(range(total))
    cov = [dict(idx=np.zeros((R // 4, C // 16), np.int8), vr=np.zeros((R, C // 16), np.int8),
                mr=np.zeros((R, C // 16), np.int8), vc=np.zeros((C, R // 16), np.int8),
                mc=np.zeros((C, R // 16), np.int8)) for R, C in shapes]
    for t in ts:
        k = max(i for i in range(len(shapes)) if t >= begin[i])
        R, C = shapes[k]
        tiles_c = cdiv(C, TILE)
        u = t - begin[k]
        ti, tj = u // tiles_c, u % tiles_c
        r0, c0 = ti * TILE, tj * TILE
        rows, cols = min(TILE, R - r0), min(TILE, C - c0)
        cv = cov[k]
        tid = np.arange(THREADS)
        if rows == TILE and cols == TILE:
            # write_full_tile: segment tid % 8 of rows (columns) tid / 8 + 32 k,
            # at offsets that must be the blocked order's
            g4, r = tid % 8, tid // 8
            np.add.at(cv["idx"], (r0 // 4 + r, c0 // 16 + g4), 1)
            pv_r, pm_r = blocked_positions(R, C // 2, VALS_BLOCK), blocked_positions(R, C // 16, META_BLOCK)
            pv_c, pm_c = blocked_positions(C, R // 2, VALS_BLOCK), blocked_positions(C, R // 16, META_BLOCK)
            for kk in range(TILE // 32):
                rr = r + 32 * kk
                assert (full_tile_form_offsets(R, C // 2, VALS_BLOCK, r0, c0 // 2, r, g4, kk)
                        == pv_r[r0 + rr, c0 // 2 + 8 * g4]).all()
                assert (full_tile_form_offsets(R, C // 16, META_BLOCK, r0, c0 // 16, r, g4, kk)
                        == pm_r[r0 + rr, c0 // 16 + g4]).all()
                assert (full_tile_form_offsets(C, R // 2, VALS_BLOCK, c0, r0 // 2, r, g4, kk)
                        == pv_c[c0 + rr, r0 // 2 + 8 * g4]).all()
                assert (full_tile_form_offsets(C, R // 16, META_BLOCK, c0, r0 // 16, r, g4, kk)
                        == pm_c[c0 + rr, r0 // 16 + g4]).all()
                np.add.at(cv["vr"], (r0 + rr, c0 // 16 + g4), 1)
                np.add.at(cv["mr"], (r0 + rr, c0 // 16 + g4), 1)
                np.add.at(cv["vc"], (c0 + rr, r0 // 16 + g4), 1)
                np.add.at(cv["mc"], (c0 + rr, r0 // 16 + g4), 1)
        else:
            # write_tile's loops over the ragged tile
            nbc, nbr = cols // 4, rows // 4
            i = np.arange(nbr * (nbc // 4))
            np.add.at(cv["idx"], (r0 // 4 + i // (nbc // 4), c0 // 16 + i % (nbc // 4)), 1)
            i = np.arange(rows * (nbc // 4))
            for key in ("vr", "mr"):
                np.add.at(cv[key], (r0 + i // (nbc // 4), c0 // 16 + i % (nbc // 4)), 1)
            i = np.arange(cols * (nbr // 4))
            for key in ("vc", "mc"):
                np.add.at(cv[key], (c0 + i // (nbr // 4), r0 // 16 + i % (nbr // 4)), 1)
    for (R, C), cv in zip(shapes, cov):
        for key, a in cv.items():
            assert (a == 1).all(), f"{key} of a {R}x{C} weight is not written exactly once"


# ----------------------------------------------------------------------------
# MVUE (sp24_mvue.hip): one workgroup of 256 lanes per 16 words (four column
# blocks) of a 64-row band

def check_mvue(rows, cols):
    """Every meta word (and its 8 halves of vals) written once, at its
    blocked-order position, and every lane's 16 entries inside the input."""
    m = cols // 16
    if rows == 0 or m == 0:
        return
    regions, bands = cdiv(m, 16), cdiv(rows, 64)
    pos = blocked_positions(rows, m, META_BLOCK)   # vals segments share meta's order
    assert (blocked_positions(rows, cols // 2, VALS_BLOCK)[:, ::8] == pos * 8).all()
    seen = np.zeros(rows * m, np.int8)
    lane, wave = np.arange(256) % 64, np.arange(256) // 64
    for b in range(bands * regions):
        band, reg = b // regions, b % regions
        r0 = 64 * band
        h = min(64, rows - r0)
        seg = 16 * reg + lane % 16
        live = seg < m
        j = seg >> 2
        w = np.minimum(4, m - 4 * j)
        blk = r0 * m + 4 * j * h + (seg & 3)
        rr = wave * 4 + lane // 16
        while True:
            ok = live & (rr < h)
            if not ok.any():
                break
            r = r0 + rr[ok]
            out = blk[ok] + rr[ok] * w[ok]
            assert (out == pos[r, seg[ok]]).all()
            assert (r * cols + 16 * seg[ok] + 16 <= rows * cols).all()
            np.add.at(seen, out, 1)
            rr = rr + 16
    assert (seen == 1).all()


# ----------------------------------------------------------------------------
# the shapes of the GPU tests and the benchmark

FFN = [WL.GPT2_355M, WL.GPT2_774M, WL.GPT2_1P5B]
GEMMS = sorted({(T, N, K) for cfg in [WL.TINY] + FFN for _, T, N, K in cfg.gemm_shapes()} | {
    (1, 16, 16), (7, 48, 80), (100, 272, 144), (129, 256, 512), (300, 528, 336), (256, 64, 4112), (300, 320, 192),
    (16347, 1152, 128), (16347, 1280, 128), (16347, 6400, 128), (16347, 128, 1152), (16347, 128, 1280),
    (16347, 128, 6400), (16384, 256, 65472), (16401, 256, 65472), (300, 272, 192), (37, 48, 80), (513, 528, 256),
    (1000, 1040, 448), (96, 160, 192), (96, 192, 160), (1, 32, 64), (100, 96, 128), (300, 544, 320),
    (257, 256, 1024), (300, 32, 64)})


@pytest.mark.parametrize("T,N,K", GEMMS)
def test_spmm_writes_and_loads(T, N, K):
    check_spmm(T, N, K)


def test_max_size_shapes_take_the_paths_their_tests_name():
    assert fast_path(16384, 256, 65472) and not fast_path(16401, 256, 65472)


@pytest.mark.parametrize("cfg", [WL.TINY] + FFN, ids=lambda c: c.name)
def test_grouped_queues_cover_every_tile_once(cfg):
    jobs = [(T, N, K) for _, T, N, K in cfg.gemm_shapes()]
    tiles = group_queues(jobs)
    want = {(q, a, b) for q, (T, N, K) in enumerate(jobs) for a in range(cdiv(N, 256)) for b in range(cdiv(T, 256))}
    assert len(tiles) == len(want) and set(tiles) == want
    # each tile of a grouped launch is a fast-path tile of its product
    for T, N, K in jobs:
        if fast_path(T, N, K) and K >= 192:
            for a in range(cdiv(N, 256)):
                check_fast_loads(256, 256, 128, 64, T, N, K, a * 256, 0)


@pytest.mark.parametrize("T,R,C", sorted({(T, R, C) for cfg in FFN for (T, R, C) in
                                          ((cfg.tokens, cfg.dff, cfg.d), (cfg.tokens, cfg.d, cfg.dff))} | {
    (1, 16, 16), (33, 272, 144), (100, 528, 336), (700, 256, 160), (64, 1040, 656), (2048, 4096, 4096),
    (16384, 65520, 16), (0, 272, 400), (16384, 1600, 3200), (16384, 4096, 5120), (1000, 6400, 1600),
    (33, 1600, 6400), (32, 6400, 1600), (976, 3072, 2560), (40, 3072, 2560), (976, 2560, 3072)}))
def test_weight_grad_writes_and_loads(T, R, C):
    check_weight_grad(T, R, C)


def test_weight_grad_splits_the_gpt2_1p5b_weights():
    assert dw_shape(16384, 6400, 1600) == (256, 320, 128, 160, True)
    assert dw_shape(16384, 1600, 6400) == (320, 256, 160, 128, True)
    assert dw_shape(32, 6400, 1600)[4] is False   # one stage of tokens: nothing to split
    assert dw_shape(16384, 1600, 3200)[4] is False   # ragged 256 x 320 tiles: not split
    assert dw_shape(16384, 4096, 5120) == (256, 320, 128, 160, False)   # one full round unsplit


@pytest.mark.parametrize("R,C,bm,bn,bound", [(6400, 1600, 256, 320, 1.75), (1600, 6400, 320, 256, 1.75),
                                              (3072, 2560, 256, 320, 2.4)])
def test_weight_grad_split_fetches_less(R, C, bm, bn, bound):
    """The split's XCD pairs fetch fewer operand bytes than the same tiles run
    whole on 8 XCDs (and than the split's earlier same-XCD pairing, which had
    each XCD fetch the strips of the whole-tile runs over all the tokens)."""
    T = 16384
    split = dw_l2_fill_bytes(T, R, C, bm, bn, True)
    whole = dw_l2_fill_bytes(T, R, C, bm, bn, False)
    assert split < 0.7 * whole
    assert split < bound * (R + C) * T * 2   # the operands themselves, (R + C) T fp16


@pytest.mark.parametrize("shapes", [[(64, 64)], [(4096, 4096)], [(6400, 1600), (1600, 6400)],
                                    [(4096, 1024), (1024, 4096)], [(5120, 1280), (1280, 5120)],
                                    [(144, 272), (272, 144), (16, 16), (512, 128), (64, 1040)], [(16, 1040)]],
                         ids=lambda s: "+".join(f"{r}x{c}" for r, c in s))
def test_search_compress_writes(shapes):
    check_search_compress(shapes)


@pytest.mark.parametrize("n,m,b", [(1, 1, 4), (3, 5, 4), (64, 32, 32), (65, 33, 32), (130, 40, 32), (200, 7, 4),
                                   (6400, 800, 32), (1600, 400, 4), (16, 2, 4), (272, 72, 32)])
def test_form_off_is_the_blocked_order(n, m, b):
    r, c = np.meshgrid(np.arange(n), np.arange(m), indexing="ij")
    assert (form_off(r, c, n, m, b) == blocked_positions(n, m, b)).all()


@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 48), (33, 256), (64, 1024), (256, 512), (100, 144), (65, 80),
                                       (16384, 6400), (2048, 1600)])
def test_mvue_writes(rows, cols):
    check_mvue(rows, cols)
