"""Host-side checks of the C ABI library: no GPU and no kernel launch needed.

* libsp24.so loads and exports every function that include/sp24.h declares;
* the pattern table compiled into the library equals the oracle's
  independently enumerated list;
* every argument error is reported before any HIP call (the pointers passed
  here are fake and would fault if the library ever used them);
* zero-sized problems succeed without touching the device.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import sp24_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sp24.h")


@pytest.fixture(scope="module")
def L():
    from structured_sparse_transformer_amd import sp24
    if not os.path.exists(sp24.LIB_PATH):
        from structured_sparse_transformer_amd import build
        build.build()
    return sp24.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sp24_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("sp24_mask_search", "sp24_compress", "sp24_search_compress", "sp24_search_compress_batch",
              "sp24_flip_count", "sp24_weight_grad", "sp24_geglu_fwd", "sp24_geglu_bwd", "sp24_mvue",
              "sp24_spmm_fwd", "sp24_spmm_fwd_geglu",
              "sp24_spmm_bwd_input", "sp24_spmm_group", "sp24_spmm_group_noalloc", "sp24_status_str",
              "sp24_pattern_table",
              "sp24_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_pattern_table_matches_oracle(L):
    from structured_sparse_transformer_amd import sp24
    got = sp24.sp24_pattern_table()
    masks = O.pattern_masks()
    want = [int(sum(int(masks[p, r, c]) << (4 * r + c) for r in range(4) for c in range(4))) for p in range(90)]
    assert got == want
    assert got[0] == 0xCC33 and got[89] == 0x33CC


def test_version_and_status_strings(L):
    assert L.sp24_abi_version() == 8
    for s in range(7):
        assert L.sp24_status_str(s)
    assert L.sp24_status_str(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)       # aligned, never dereferenced
MIS = ctypes.c_void_p(0x1008)        # 8-byte aligned only
NUL = None


def test_mask_search_validation(L):
    f = L.sp24_mask_search
    assert f(FAKE, 6, 8, FAKE, NUL) == 2          # R not a multiple of 4
    assert f(FAKE, 8, 10, FAKE, NUL) == 2
    assert f(FAKE, -4, 8, FAKE, NUL) == 2
    assert f(NUL, 8, 8, FAKE, NUL) == 1
    assert f(FAKE, 8, 8, NUL, NUL) == 1
    assert f(MIS, 8, 8, FAKE, NUL) == 3
    assert f(FAKE, 8, 8, MIS, NUL) == 3
    assert f(FAKE, 1 << 31, 8, FAKE, NUL) == 6
    assert f(FAKE, 1 << 24, 1 << 20, FAKE, NUL) == 6
    assert f(NUL, 0, 8, NUL, NUL) == 0            # empty: nothing to do
    assert f(NUL, 8, 0, NUL, NUL) == 0


def test_compress_validation(L):
    f = L.sp24_compress
    assert f(FAKE, FAKE, 8, 16, FAKE, FAKE, FAKE, FAKE, NUL) == 2       # R % 16
    assert f(FAKE, FAKE, 16, 20, FAKE, FAKE, FAKE, FAKE, NUL) == 2
    assert f(FAKE, NUL, 16, 16, FAKE, FAKE, FAKE, FAKE, NUL) == 1       # idx required
    assert f(FAKE, FAKE, 16, 16, NUL, NUL, NUL, NUL, NUL) == 1          # no output at all
    assert f(FAKE, FAKE, 16, 16, FAKE, NUL, NUL, NUL, NUL) == 1         # half a pair
    assert f(FAKE, FAKE, 16, 16, NUL, NUL, NUL, FAKE, NUL) == 1
    assert f(NUL, FAKE, 16, 16, FAKE, FAKE, NUL, NUL, NUL) == 1
    assert f(MIS, FAKE, 16, 16, FAKE, FAKE, NUL, NUL, NUL) == 3
    assert f(FAKE, FAKE, 16, 16, FAKE, MIS, NUL, NUL, NUL) == 3
    assert f(NUL, NUL, 0, 16, FAKE, FAKE, NUL, NUL, NUL) == 0


def test_search_compress_validation(L):
    f = L.sp24_search_compress
    assert f(FAKE, 16, 24, FAKE, FAKE, FAKE, FAKE, FAKE, NUL) == 2
    assert f(FAKE, 16, 16, FAKE, NUL, NUL, NUL, NUL, NUL) == 1
    assert f(FAKE, 16, 16, MIS, FAKE, FAKE, NUL, NUL, NUL) == 3
    assert f(NUL, 0, 0, NUL, FAKE, FAKE, NUL, NUL, NUL) == 0


@pytest.mark.parametrize("name", ["sp24_spmm_fwd", "sp24_spmm_bwd_input"])
def test_spmm_validation(L, name):
    f = getattr(L, name)
    assert f(FAKE, FAKE, FAKE, 8, 16, 20, FAKE, NUL) == 2      # C % 16
    assert f(FAKE, FAKE, FAKE, 8, 20, 16, FAKE, NUL) == 2      # R % 16
    assert f(FAKE, FAKE, FAKE, -1, 16, 16, FAKE, NUL) == 2
    assert f(NUL, FAKE, FAKE, 8, 16, 16, FAKE, NUL) == 1
    assert f(FAKE, NUL, FAKE, 8, 16, 16, FAKE, NUL) == 1
    assert f(FAKE, FAKE, NUL, 8, 16, 16, FAKE, NUL) == 1
    assert f(FAKE, FAKE, FAKE, 8, 16, 16, NUL, NUL) == 1
    assert f(FAKE, FAKE, FAKE, 8, 16, 16, MIS, NUL) == 3
    assert f(MIS, FAKE, FAKE, 8, 16, 16, FAKE, NUL) == 3
    assert f(FAKE, FAKE, FAKE, 1 << 31, 16, 16, FAKE, NUL) == 6
    assert f(NUL, NUL, NUL, 0, 16, 16, NUL, NUL) == 0          # no tokens
    assert f(NUL, NUL, NUL, 8, 0, 0, NUL, NUL) == 0


def test_binding_refuses_cpu_tensors(L):
    torch = pytest.importorskip("torch")
    from structured_sparse_transformer_amd import sp24
    with pytest.raises(ValueError):
        sp24.sp24_mask_search(torch.zeros(8, 8, dtype=torch.float16))


def test_search_compress_batch_validation(L):
    from structured_sparse_transformer_amd.sp24 import ScJob
    f = L.sp24_search_compress_batch
    ok = ScJob(0x1000, 16, 16, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000)
    arr = (ScJob * 9)(*([ok] * 9))
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert f(None, 1, NUL) == 1
    assert f(p, 0, NUL) == 2
    assert f(p, 9, NUL) == 2
    bad_shape = (ScJob * 2)(ok, ScJob(0x1000, 16, 20, None, 0x3000, 0x4000, None, None))
    assert f(ctypes.cast(bad_shape, ctypes.c_void_p), 2, NUL) == 2      # second job checked before launching
    half = (ScJob * 1)(ScJob(0x1000, 16, 16, None, 0x3000, None, None, None))
    assert f(ctypes.cast(half, ctypes.c_void_p), 1, NUL) == 1
    mis = (ScJob * 1)(ScJob(0x1008, 16, 16, None, 0x3000, 0x4000, None, None))
    assert f(ctypes.cast(mis, ctypes.c_void_p), 1, NUL) == 3
    empty = (ScJob * 2)(ScJob(None, 0, 16, None, 0x3000, 0x4000, None, None),
                        ScJob(None, 16, 0, None, 0x3000, 0x4000, None, None))
    assert f(ctypes.cast(empty, ctypes.c_void_p), 2, NUL) == 0         # all empty: nothing launched


def test_search_compress_batch_flip_validation(L):
    from structured_sparse_transformer_amd.sp24 import ScJob
    f = L.sp24_search_compress_batch
    base = (0x1000, 16, 16, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000)
    one = lambda *extra: ctypes.cast((ScJob * 1)(ScJob(*base, *extra)), ctypes.c_void_p)  # noqa: E731
    assert f(one(0x7000, None), 1, NUL) == 1          # previous masks without a counter
    assert f(one(None, 0x8000), 1, NUL) == 1          # counter without previous masks
    assert f(one(0x7008, 0x8000), 1, NUL) == 3        # idx_prev needs 16 bytes
    assert f(one(0x7000, 0x8004), 1, NUL) == 3        # the counter needs 8
    empty = (ScJob * 1)(ScJob(None, 0, 16, None, 0x3000, 0x4000, None, None, 0x7000, 0x8008))
    assert f(ctypes.cast(empty, ctypes.c_void_p), 1, NUL) == 0


def test_flip_count_validation(L):
    f = L.sp24_flip_count
    assert f(FAKE, FAKE, -1, FAKE, NUL) == 2
    assert f(FAKE, FAKE, 1 << 40, FAKE, NUL) == 6
    assert f(NUL, FAKE, 4, FAKE, NUL) == 1
    assert f(FAKE, NUL, 4, FAKE, NUL) == 1
    assert f(FAKE, FAKE, 4, NUL, NUL) == 1
    assert f(MIS, FAKE, 4, FAKE, NUL) == 3
    assert f(FAKE, MIS, 4, FAKE, NUL) == 3
    assert f(FAKE, FAKE, 4, ctypes.c_void_p(0x1004), NUL) == 3
    assert f(NUL, NUL, 0, NUL, NUL) == 0


def test_weight_grad_validation(L):
    f = L.sp24_weight_grad
    c = ctypes.c_float(0.5)
    assert f(FAKE, FAKE, FAKE, FAKE, c, 8, 16, 20, FAKE, NUL) == 2          # C % 16
    assert f(FAKE, FAKE, FAKE, FAKE, c, -1, 16, 16, FAKE, NUL) == 2
    assert f(FAKE, FAKE, FAKE, NUL, c, 8, 16, 16, FAKE, NUL) == 1           # W without idx
    assert f(FAKE, FAKE, NUL, FAKE, c, 8, 16, 16, FAKE, NUL) == 1
    assert f(NUL, FAKE, NUL, NUL, c, 8, 16, 16, FAKE, NUL) == 1
    assert f(FAKE, FAKE, NUL, NUL, c, 8, 16, 16, NUL, NUL) == 1
    assert f(MIS, FAKE, NUL, NUL, c, 8, 16, 16, FAKE, NUL) == 3
    assert f(FAKE, FAKE, NUL, NUL, c, 8, 16, 16, MIS, NUL) == 3
    assert f(FAKE, FAKE, MIS, FAKE, c, 8, 16, 16, FAKE, NUL) == 3
    assert f(FAKE, FAKE, NUL, NUL, c, 1 << 20, 1024, 16, FAKE, NUL) == 6    # T*R >= 2^30
    assert f(FAKE, FAKE, NUL, NUL, c, 1 << 20, 16, 1024, FAKE, NUL) == 6
    assert f(NUL, NUL, NUL, NUL, c, 8, 0, 16, NUL, NUL) == 0                # empty output


def test_geglu_validation(L):
    fw, bw = L.sp24_geglu_fwd, L.sp24_geglu_bwd
    assert fw(FAKE, 4, 12, 4, FAKE, NUL) == 2          # h % 8
    assert fw(FAKE, 4, 16, 4, FAKE, NUL) == 2          # group % 8
    assert fw(FAKE, 4, 24, 16, FAKE, NUL) == 2         # h % group
    assert fw(FAKE, 4, 16, 0, FAKE, NUL) == 2
    assert fw(FAKE, -1, 16, 8, FAKE, NUL) == 2
    assert fw(NUL, 4, 16, 8, FAKE, NUL) == 1
    assert fw(FAKE, 4, 16, 8, MIS, NUL) == 3
    assert fw(FAKE, 1 << 30, 1 << 10, 8, FAKE, NUL) == 6
    # one launch takes at most 2^32 - 256 work-items of 8 units each
    assert fw(FAKE, 1 << 20, (1 << 15) - 16, 8, MIS, NUL) == 3       # 2^32 - 2^21 items: allowed
    assert fw(FAKE, 1 << 20, 1 << 15, 8, FAKE, NUL) == 6             # 2^32 items
    assert bw(FAKE, FAKE, (1 << 32) // 2048 - 1, 2048 * 8, 8, MIS, NUL) == 3   # 2^32 - 2048 items: allowed
    assert bw(FAKE, FAKE, 1 << 21, 2048 * 8, 8, FAKE, NUL) == 6
    assert fw(NUL, 0, 16, 8, NUL, NUL) == 0
    assert bw(FAKE, NUL, 4, 16, 8, FAKE, NUL) == 1
    assert bw(FAKE, FAKE, 4, 16, 8, MIS, NUL) == 3
    assert bw(FAKE, FAKE, 4, 20, 8, FAKE, NUL) == 2
    assert bw(NUL, NUL, 4, 0, 8, NUL, NUL) == 0


def test_mvue_validation(L):
    f = L.sp24_mvue
    assert f(FAKE, FAKE, 4, 24, FAKE, FAKE, NUL) == 2           # cols % 16
    assert f(FAKE, FAKE, -1, 16, FAKE, FAKE, NUL) == 2
    assert f(NUL, FAKE, 4, 16, FAKE, FAKE, NUL) == 1
    assert f(FAKE, NUL, 4, 16, FAKE, FAKE, NUL) == 1
    assert f(FAKE, FAKE, 4, 16, FAKE, NUL, NUL) == 1
    assert f(FAKE, MIS, 4, 16, FAKE, FAKE, NUL) == 3
    assert f(FAKE, FAKE, 1 << 31, 16, FAKE, FAKE, NUL) == 6
    # one workgroup of 256 work-items per 64 x 256 panel, at most 2^32 - 256 work-items per launch
    assert f(FAKE, FAKE, (1 << 30) - 64, 256, MIS, FAKE, NUL) == 3   # 2^24 - 1 panels: allowed
    assert f(FAKE, FAKE, (1 << 30) - 63, 256, FAKE, FAKE, NUL) == 6  # a 2^24-th (partial) band
    assert f(FAKE, FAKE, 1 << 29, 512, FAKE, FAKE, NUL) == 6         # 2^23 bands of 2 panels
    assert f(FAKE, FAKE, 1 << 29, 272, MIS, FAKE, NUL) == 6          # 272 columns take 2 panels
    assert f(FAKE, FAKE, (1 << 29) - 64, 512, MIS, FAKE, NUL) == 3   # 2^23 - 1 bands of 2 panels
    assert f(NUL, NUL, 0, 16, NUL, NUL, NUL) == 0


def test_spmm_fwd_geglu_validation(L):
    f = L.sp24_spmm_fwd_geglu
    assert f(FAKE, FAKE, FAKE, 8, 48, 64, NUL, FAKE, NUL) == 2      # R % 32
    assert f(FAKE, FAKE, FAKE, 8, 64, 20, NUL, FAKE, NUL) == 2      # C % 16
    assert f(FAKE, FAKE, FAKE, -1, 64, 64, NUL, FAKE, NUL) == 2
    assert f(FAKE, FAKE, FAKE, 8, 64, 64, NUL, NUL, NUL) == 1
    assert f(NUL, FAKE, FAKE, 8, 64, 64, NUL, FAKE, NUL) == 1
    assert f(FAKE, FAKE, FAKE, 8, 64, 64, MIS, FAKE, NUL) == 3
    assert f(FAKE, FAKE, FAKE, 8, 64, 64, NUL, MIS, NUL) == 3
    assert f(NUL, NUL, NUL, 0, 64, 64, NUL, NUL, NUL) == 0
    # T * R/16 work-items of the GEGLU kernel that finishes unfused shapes
    assert f(FAKE, FAKE, FAKE, 1 << 20, 1 << 16, 16, NUL, FAKE, NUL) == 6
    assert f(FAKE, FAKE, FAKE, 1 << 20, (1 << 16) - 32, 16, NUL, MIS, NUL) == 3


def test_spmm_group_validation(L):
    from structured_sparse_transformer_amd.sp24 import Gemm
    f = L.sp24_spmm_group

    def arr(*gs):
        a = (Gemm * len(gs))()
        for k, g in enumerate(gs):
            a[k] = g
        return ctypes.cast(a, ctypes.c_void_p)

    ok = Gemm(0x1000, 0x1000, 0x1000, 0x1000, 300, 256, 1600)
    assert f(None, 1, FAKE, NUL) == 1
    assert f(arr(ok), 0, FAKE, NUL) == 2                                    # count outside 1..8
    assert f(arr(*([ok] * 9)), 9, FAKE, NUL) == 2
    assert f(arr(ok), 1, NUL, NUL) == 1                                     # no workspace
    assert f(arr(ok), 1, MIS, NUL) == 3
    assert f(arr(ok, Gemm(0x1000, 0x1000, 0x1000, 0x1000, 300, 250, 1600)), 2, FAKE, NUL) == 2   # N % 16
    assert f(arr(ok, Gemm(0x1000, 0x1000, 0x1000, 0x1000, -1, 256, 64)), 2, FAKE, NUL) == 2
    assert f(arr(ok, Gemm(0x1000, 0, 0x1000, 0x1000, 300, 256, 64)), 2, FAKE, NUL) == 1
    assert f(arr(ok, Gemm(0x1000, 0x1000, 0x1000, 0x1008, 300, 256, 64)), 2, FAKE, NUL) == 3
    assert f(arr(ok, Gemm(0x1000, 0x1000, 0x1000, 0x1000, 1 << 31, 16, 16)), 2, FAKE, NUL) == 6
    # every product is checked before anything is launched; empty products need no buffers
    assert f(arr(Gemm(0, 0, 0, 0, 0, 256, 64), Gemm(0, 0, 0, 0, 16, 0, 64)), 2, FAKE, NUL) == 0
    # the allocation-free variant checks the same way (and needs no workspace)
    g = L.sp24_spmm_group_noalloc
    assert g(None, 1, NUL) == 1
    assert g(arr(*([ok] * 9)), 9, NUL) == 2
    assert g(arr(ok, Gemm(0x1000, 0x1000, 0x1000, 0x1000, 300, 250, 1600)), 2, NUL) == 2
    assert g(arr(ok, Gemm(0x1000, 0x1000, 0x1000, 0x1008, 300, 256, 64)), 2, NUL) == 3


def test_ffn_layer_rejects_bad_shapes():
    """SparseGegluFFN checks its weights' shapes before any device work."""
    torch = pytest.importorskip("torch")
    from structured_sparse_transformer_amd.ffn import SparseGegluFFN
    w1 = torch.zeros(64, 32, dtype=torch.float16)
    SparseGegluFFN(w1, torch.zeros(32, 32, dtype=torch.float16))    # [2h, d] and [d, h], 2h = 64
    with pytest.raises(ValueError):
        SparseGegluFFN(w1, torch.zeros(32, 64, dtype=torch.float16))   # W2 must be [d, h]
    with pytest.raises(ValueError):
        SparseGegluFFN(torch.zeros(48, 32, dtype=torch.float16), torch.zeros(32, 24, dtype=torch.float16))
    layer = SparseGegluFFN(w1, torch.zeros(32, 32, dtype=torch.float16))
    with pytest.raises(RuntimeError, match="refresh"):
        layer.forward(torch.zeros(8, 32, dtype=torch.float16))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 ends with a message before any GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_binding_checks_operand_shapes_before_any_pointer():
    """The C ABI takes plain pointers, so the binding must refuse an operand
    whose shape or dtype disagrees with the sizes passed beside it: the
    kernels would otherwise read past its end.  The checks run before any
    pointer is taken, so CPU tensors are enough to exercise them."""
    torch = pytest.importorskip("torch")
    from structured_sparse_transformer_amd import sp24 as sp
    h = lambda *s: torch.zeros(*s, dtype=torch.float16)   # noqa: E731
    i16 = lambda *s: torch.zeros(*s, dtype=torch.int16)   # noqa: E731
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)    # noqa: E731
    R, C, T = 64, 32, 8
    good = (h(R, C // 2), i16(R, C // 16))
    bad_forms = [(h(R, C // 2 - 8), good[1]), (good[0], i16(R - 16, C // 16)),
                 (good[0].float(), good[1]), (good[0], good[1].to(torch.int32)), (None, good[1])]
    for vals, meta in bad_forms:
        with pytest.raises(ValueError):
            sp.sp24_spmm_fwd(h(T, C), vals, meta, R, C)
        with pytest.raises(ValueError):
            sp.sp24_spmm_fwd_geglu(h(T, C), vals, meta, R, C)
    with pytest.raises(ValueError):       # column form of the same weight is [C, R/2]
        sp.sp24_spmm_bwd_input(h(T, R), h(R, C // 2), i16(R, C // 16), R, C)
    with pytest.raises(ValueError):       # a dimension that is not a multiple of 16
        sp.sp24_spmm_fwd(h(T, 40), h(R, 20), i16(R, 2), R, 40)
    with pytest.raises(ValueError):
        sp.sp24_compress(h(R, C), u8(R // 4, C // 4 - 1))
    with pytest.raises(ValueError):
        sp.sp24_weight_grad(h(T, R), h(T, C), h(R, C), u8(R // 4 + 1, C // 4))
    with pytest.raises(ValueError):
        sp.sp24_search_compress_batch([h(R, C)], prev=[u8(R // 4, C // 4 + 4)],
                                      flips=[torch.zeros(1, dtype=torch.int64)])
    # well-formed operands get past the checks and stop at the device test
    with pytest.raises(ValueError, match="on the GPU"):
        sp.sp24_spmm_fwd(h(T, C), *good, R, C)
