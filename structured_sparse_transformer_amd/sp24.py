"""ctypes binding of libsp24.so (argument marshalling only).

Each function takes and returns torch tensors on the current HIP device; the
C library does all of the computing, on the caller's current torch stream.
Output tensors are allocated with torch when not supplied.  Errors from the
library raise :class:`Sp24Error`.  There is no fallback: without the built
library every call raises.

Shapes and layouts follow ``include/sp24.h``: W is fp16 [R, C]; idx uint8
[R/4, C/4]; the row form is (vals_row fp16 [R, C/2], meta_row int16 [R, C/16])
and the column form (vals_col fp16 [C, R/2], meta_col int16 [C, R/16]).  torch
has no uint16, so meta words travel as int16 tensors with the same bits.  The
forms' tensors carry those logical shapes, but their elements are in the
header's blocked order (64-row bands of contiguous column blocks), so a row
of such a tensor is not a row of the form.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsp24.so")

SP24_OK = 0
STATUS_NAMES = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_ALIGN", 4: "ERR_LAUNCH",
                5: "ERR_UNSUPPORTED", 6: "ERR_TOO_LARGE"}
EXPORTS = ("sp24_mask_search", "sp24_compress", "sp24_search_compress", "sp24_search_compress_batch",
           "sp24_flip_count", "sp24_weight_grad", "sp24_geglu_fwd", "sp24_geglu_bwd", "sp24_mvue",
           "sp24_spmm_fwd", "sp24_spmm_fwd_geglu", "sp24_spmm_bwd_input", "sp24_spmm_group",
           "sp24_spmm_group_noalloc", "sp24_status_str",
           "sp24_pattern_table", "sp24_abi_version")
MAX_BATCH = 8
MAX_GROUP = 8
GROUP_WORKSPACE_BYTES = 64


class ScJob(ctypes.Structure):
    """Mirror of sp24_sc_job (include/sp24.h)."""
    _fields_ = [("W", ctypes.c_void_p), ("R", ctypes.c_int64), ("C", ctypes.c_int64), ("idx", ctypes.c_void_p),
                ("vals_row", ctypes.c_void_p), ("meta_row", ctypes.c_void_p),
                ("vals_col", ctypes.c_void_p), ("meta_col", ctypes.c_void_p),
                ("idx_prev", ctypes.c_void_p), ("flips", ctypes.c_void_p)]


class Gemm(ctypes.Structure):
    """Mirror of sp24_gemm (include/sp24.h)."""
    _fields_ = [("A", ctypes.c_void_p), ("vals", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("T", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class Sp24Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libsp24.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m structured_sparse_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "sp24_mask_search": [p, i64, i64, p, p],
            "sp24_compress": [p, p, i64, i64, p, p, p, p, p],
            "sp24_search_compress": [p, i64, i64, p, p, p, p, p, p],
            "sp24_search_compress_batch": [p, i32, p],
            "sp24_flip_count": [p, p, i64, p, p],
            "sp24_weight_grad": [p, p, p, p, ctypes.c_float, i64, i64, i64, p, p],
            "sp24_geglu_fwd": [p, i64, i64, i64, p, p],
            "sp24_geglu_bwd": [p, p, i64, i64, i64, p, p],
            "sp24_mvue": [p, p, i64, i64, p, p, p],
            "sp24_spmm_fwd": [p, p, p, i64, i64, i64, p, p],
            "sp24_spmm_fwd_geglu": [p, p, p, i64, i64, i64, p, p, p],
            "sp24_spmm_bwd_input": [p, p, p, i64, i64, i64, p, p],
            "sp24_spmm_group": [p, i32, p, p],
            "sp24_spmm_group_noalloc": [p, i32, p],
            "sp24_status_str": [i32],
            "sp24_pattern_table": [p],
            "sp24_abi_version": [],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "sp24_status_str" else i32
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != SP24_OK:
        raise Sp24Error(fn, status, lib().sp24_status_str(status).decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    # the library launches on the current device (and its current stream)
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor is on {t.device} but the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    if s.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {s.device} but the current device is cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(s.cuda_stream)


def _out(t, shape, dtype, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"output must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


def _need(t, shape, dtype, name):
    """An input tensor the library reads through a plain pointer: its shape and
    dtype must be exactly what the sizes passed alongside it imply, or the
    kernels would read past its end."""
    if t is None or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        got = "None" if t is None else f"{t.dtype} {tuple(t.shape)}"
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {got}")
    return t


def _row_form(vals, meta, R, C, name):
    """The 2:4 form of an [R, C] matrix: vals fp16 [R, C/2], meta int16 [R, C/16]."""
    if R % 16 or C % 16:
        raise ValueError(f"{name}: both dimensions must be multiples of 16, got {R} x {C}")
    _need(vals, (R, C // 2), torch.float16, f"{name} values")
    _need(meta, (R, C // 16), torch.int16, f"{name} metadata")


def _w(W):
    if W.dtype != torch.float16 or W.dim() != 2:
        raise ValueError("W must be a 2-D float16 tensor")
    return W.shape


def sp24_mask_search(W, idx=None, stream=None):
    """idx[R/4, C/4] (uint8) of the transposable pattern kept by each 4x4 block."""
    R, C = _w(W)
    idx = _out(idx, (R // 4, C // 4), torch.uint8, W.device)
    _check("sp24_mask_search", lib().sp24_mask_search(_ptr(W), R, C, _ptr(idx), _stream(stream)))
    return idx


def _forms(R, C, device, row, col, out):
    out = dict(out or {})
    if row:
        out["vals_row"] = _out(out.get("vals_row"), (R, C // 2), torch.float16, device)
        out["meta_row"] = _out(out.get("meta_row"), (R, C // 16), torch.int16, device)
    if col:
        out["vals_col"] = _out(out.get("vals_col"), (C, R // 2), torch.float16, device)
        out["meta_col"] = _out(out.get("meta_col"), (C, R // 16), torch.int16, device)
    return out


def sp24_compress(W, idx, row=True, col=True, out=None, stream=None):
    """Row and/or column 2:4 forms of W pruned by the masks ``idx``."""
    R, C = _w(W)
    _need(idx, (R // 4, C // 4), torch.uint8, "idx")
    o = _forms(R, C, W.device, row, col, out)
    _check("sp24_compress", lib().sp24_compress(
        _ptr(W), _ptr(idx), R, C, _ptr(o.get("vals_row")), _ptr(o.get("meta_row")),
        _ptr(o.get("vals_col")), _ptr(o.get("meta_col")), _stream(stream)))
    return o


def sp24_search_compress(W, want_idx=True, row=True, col=True, out=None, stream=None):
    """Mask search and compression in one pass over W."""
    R, C = _w(W)
    o = _forms(R, C, W.device, row, col, out)
    if want_idx:
        o["idx"] = _out(o.get("idx"), (R // 4, C // 4), torch.uint8, W.device)
    _check("sp24_search_compress", lib().sp24_search_compress(
        _ptr(W), R, C, _ptr(o.get("idx")), _ptr(o.get("vals_row")), _ptr(o.get("meta_row")),
        _ptr(o.get("vals_col")), _ptr(o.get("meta_col")), _stream(stream)))
    return o


def _flip_counter(f):
    """A uint64 flip counter travels as an int64 tensor view of one element."""
    if f is None:
        return None
    if f.dtype != torch.int64 or f.numel() != 1:
        raise ValueError("a flip counter is a one-element int64 tensor (or a view of one)")
    return _ptr(f).value


def sp24_search_compress_batch(Ws, outs=None, want_idx=True, row=True, col=True, prev=None, flips=None,
                               stream=None):
    """sp24_search_compress for several weights in one launch; returns one dict per weight.

    ``prev[k]`` (uint8 [R/4, C/4]) and ``flips[k]`` (a one-element int64 tensor)
    make weight k count its flipped mask entries against ``prev[k]``: the
    count is ADDED to ``flips[k]``.  ``prev[k]`` may be the weight's own
    ``outs[k]["idx"]``, which is then updated in place.
    """
    if not 1 <= len(Ws) <= MAX_BATCH:
        raise ValueError(f"between 1 and {MAX_BATCH} weights per batch")
    outs = list(outs) if outs is not None else [None] * len(Ws)
    prev = list(prev) if prev is not None else [None] * len(Ws)
    flips = list(flips) if flips is not None else [None] * len(Ws)
    if len(prev) != len(Ws) or len(flips) != len(Ws):
        raise ValueError("prev and flips need one entry per weight")
    res, jobs = [], (ScJob * len(Ws))()
    for k, W in enumerate(Ws):
        R, C = _w(W)
        o = _forms(R, C, W.device, row, col, outs[k])
        if want_idx:
            o["idx"] = _out(o.get("idx"), (R // 4, C // 4), torch.uint8, W.device)
        ptr = lambda t: _ptr(t).value if t is not None and t.numel() else None  # noqa: E731
        if prev[k] is not None:
            _need(prev[k], (R // 4, C // 4), torch.uint8, "prev")
        jobs[k] = ScJob(ptr(W), R, C, ptr(o.get("idx")), ptr(o.get("vals_row")), ptr(o.get("meta_row")),
                        ptr(o.get("vals_col")), ptr(o.get("meta_col")), ptr(prev[k]), _flip_counter(flips[k]))
        res.append(o)
    _check("sp24_search_compress_batch",
           lib().sp24_search_compress_batch(ctypes.cast(jobs, ctypes.c_void_p), len(Ws), _stream(stream)))
    return res


def sp24_flip_count(idx_prev, idx_new, flips=None, stream=None):
    """Adds to ``flips`` (a one-element int64 tensor, zeroed when not given)
    the number of mask entries that differ between the two index arrays."""
    if idx_prev.dtype != torch.uint8 or idx_new.dtype != torch.uint8 or idx_prev.shape != idx_new.shape:
        raise ValueError("idx_prev and idx_new must be uint8 tensors of one shape")
    if flips is None:
        flips = torch.zeros(1, dtype=torch.int64, device=idx_new.device)
    _check("sp24_flip_count", lib().sp24_flip_count(_ptr(idx_prev), _ptr(idx_new), idx_new.numel(),
                                                    _flip_counter(flips), _stream(stream)))
    return flips


def sp24_weight_grad(dY, X, W=None, idx=None, decay=0.0, dW=None, stream=None):
    """dW[R, C] (float32) = dY^T X + decay * (1 - M) * W, M the masks ``idx``."""
    T, R = dY.shape
    C = X.shape[1]
    if dY.dtype != torch.float16 or X.dtype != torch.float16 or X.dim() != 2 or X.shape[0] != T:
        raise ValueError("dY and X must be float16 [T, R] and [T, C]")
    if W is not None:
        _need(W, (R, C), torch.float16, "W")
    if idx is not None:
        _need(idx, (R // 4, C // 4), torch.uint8, "idx")
    dW = _out(dW, (R, C), torch.float32, dY.device)
    _check("sp24_weight_grad", lib().sp24_weight_grad(_ptr(dY), _ptr(X), _ptr(W), _ptr(idx), float(decay), T, R, C,
                                                      _ptr(dW), _stream(stream)))
    return dW


def _geglu_shape(U, group):
    if U.dtype != torch.float16 or U.dim() != 2 or U.shape[1] % 2:
        raise ValueError("U must be float16 [T, 2h]")
    T, h = U.shape[0], U.shape[1] // 2
    group = h if group is None else group
    return T, h, group


def sp24_geglu_fwd(U, group=None, out=None, stream=None):
    """out [T, h] = value * GELU(gate); U's columns in blocks of `group`
    values then `group` gates (default: the two halves)."""
    T, h, group = _geglu_shape(U, group)
    out = _out(out, (T, h), torch.float16, U.device)
    _check("sp24_geglu_fwd", lib().sp24_geglu_fwd(_ptr(U), T, h, group, _ptr(out), _stream(stream)))
    return out


def sp24_geglu_bwd(U, dout, group=None, dU=None, stream=None):
    """dU [T, 2h] in U's layout from dout [T, h]."""
    T, h, group = _geglu_shape(U, group)
    if dout.dtype != torch.float16 or tuple(dout.shape) != (T, h):
        raise ValueError("dout must be float16 [T, h]")
    dU = _out(dU, (T, 2 * h), torch.float16, U.device)
    _check("sp24_geglu_bwd", lib().sp24_geglu_bwd(_ptr(U), _ptr(dout), T, h, group, _ptr(dU), _stream(stream)))
    return dU


def sp24_mvue(M, U, out=None, stream=None):
    """MVUE 2:4 estimate of M (fp16 [rows, cols]) with uniforms U (fp32
    [rows, cols/4]); returns {"vals": fp16 [rows, cols/2], "meta": int16
    [rows, cols/16]}."""
    if M.dtype != torch.float16 or M.dim() != 2:
        raise ValueError("M must be a 2-D float16 tensor")
    rows, cols = M.shape
    if U.dtype != torch.float32 or tuple(U.shape) != (rows, cols // 4):
        raise ValueError("U must be float32 [rows, cols/4]")
    out = dict(out or {})
    out["vals"] = _out(out.get("vals"), (rows, cols // 2), torch.float16, M.device)
    out["meta"] = _out(out.get("meta"), (rows, cols // 16), torch.int16, M.device)
    _check("sp24_mvue", lib().sp24_mvue(_ptr(M), _ptr(U), rows, cols, _ptr(out["vals"]), _ptr(out["meta"]),
                                        _stream(stream)))
    return out


def sp24_spmm_fwd(X, vals_row, meta_row, R, C, Y=None, stream=None):
    """Y[T, R] = X[T, C] * Ws^T."""
    T = X.shape[0]
    if X.dtype != torch.float16 or tuple(X.shape) != (T, C):
        raise ValueError("X must be float16 [T, C]")
    _row_form(vals_row, meta_row, R, C, "the row form")
    Y = _out(Y, (T, R), torch.float16, X.device)
    _check("sp24_spmm_fwd", lib().sp24_spmm_fwd(_ptr(X), _ptr(vals_row), _ptr(meta_row), T, R, C,
                                                _ptr(Y), _stream(stream)))
    return Y


def sp24_spmm_fwd_geglu(X, vals_row, meta_row, R, C, out=None, U=False, stream=None):
    """out[T, R/2] = value * GELU(gate) of U = X * Ws^T, W's rows in blocks of
    16 values then their 16 gates.  U=True also returns the products [T, R]
    (a tensor may be passed instead); returns (out, U or None)."""
    T = X.shape[0]
    if X.dtype != torch.float16 or tuple(X.shape) != (T, C):
        raise ValueError("X must be float16 [T, C]")
    _row_form(vals_row, meta_row, R, C, "the row form")
    out = _out(out, (T, R // 2), torch.float16, X.device)
    if U is True:
        U = torch.empty(T, R, dtype=torch.float16, device=X.device)
    elif U is False or U is None:
        U = None
    else:
        U = _out(U, (T, R), torch.float16, X.device)
    _check("sp24_spmm_fwd_geglu", lib().sp24_spmm_fwd_geglu(_ptr(X), _ptr(vals_row), _ptr(meta_row), T, R, C,
                                                            _ptr(U), _ptr(out), _stream(stream)))
    return out, U


def sp24_spmm_bwd_input(dY, vals_col, meta_col, R, C, dX=None, stream=None):
    """dX[T, C] = dY[T, R] * Ws."""
    T = dY.shape[0]
    if dY.dtype != torch.float16 or tuple(dY.shape) != (T, R):
        raise ValueError("dY must be float16 [T, R]")
    _row_form(vals_col, meta_col, C, R, "the column form")
    dX = _out(dX, (T, C), torch.float16, dY.device)
    _check("sp24_spmm_bwd_input", lib().sp24_spmm_bwd_input(_ptr(dY), _ptr(vals_col), _ptr(meta_col), T, R, C,
                                                            _ptr(dX), _stream(stream)))
    return dX


def sp24_pattern_table():
    """The 90 patterns as 16-bit masks (bit 4r+c for kept entry (r, c))."""
    buf = (ctypes.c_uint16 * 90)()
    _check("sp24_pattern_table", lib().sp24_pattern_table(ctypes.cast(buf, ctypes.c_void_p)))
    return list(buf)


_group_ws = {}


def group_workspace(device=None):
    """The binding's workspace for sp24_spmm_group on a device: zeroed once,
    and left zero by every call that completes.  Calls that overlap in time
    (on different streams) must pass workspaces of their own."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else torch.device(device).index)
    ws = _group_ws.get(dev.index)
    if ws is None:
        ws = torch.zeros(GROUP_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev)
        _group_ws[dev.index] = ws
    return ws


def _gemm_descs(gemms):
    if not 1 <= len(gemms) <= MAX_GROUP:
        raise ValueError(f"between 1 and {MAX_GROUP} products per group")
    descs, outs = (Gemm * len(gemms))(), []
    for k, (A, vals, meta, out) in enumerate(gemms):
        if A.dtype != torch.float16 or A.dim() != 2:
            raise ValueError("A must be a 2-D float16 tensor")
        T, K = A.shape
        if vals.dim() != 2:
            raise ValueError("vals must be 2-D")
        N = vals.shape[0]
        _row_form(vals, meta, N, K, f"product {k}")
        out = _out(out, (T, N), torch.float16, A.device)
        outs.append(out)
        ptr = lambda t: _ptr(t).value if t is not None and t.numel() else None  # noqa: E731
        descs[k] = Gemm(ptr(A), ptr(vals), ptr(meta), ptr(out), T, N, K)
    return descs, outs


def sp24_spmm_group_noalloc(gemms, stream=None):
    """sp24_spmm_group with the library's own per-GPU queue counters instead
    of a workspace (the C entry point allocates nothing).  Calls that overlap
    in time on one GPU race.  Output tensors given as None are allocated here
    by torch; pass them all to keep the whole call allocation-free."""
    descs, outs = _gemm_descs(gemms)
    _check("sp24_spmm_group_noalloc", lib().sp24_spmm_group_noalloc(ctypes.cast(descs, ctypes.c_void_p), len(gemms),
                                                                    _stream(stream)))
    return outs


def sp24_spmm_group(gemms, workspace=None, stream=None):
    """Several independent products out = A * S^T in one launch.

    ``gemms`` is a list of (A, vals, meta, out) with A fp16 [T, K], (vals,
    meta) the 2:4 row form of S [N, K] (fp16 [N, K/2], int16 [N, K/16]) and
    out fp16 [T, N] or None (allocated).  The forward product of a layer is
    (X, vals_row, meta_row, Y); its input gradient (dY, vals_col, meta_col,
    dX).  Returns the outputs."""
    descs, outs = _gemm_descs(gemms)
    ws = group_workspace() if workspace is None else workspace
    if ws.numel() * ws.element_size() < GROUP_WORKSPACE_BYTES:
        raise ValueError(f"the workspace needs {GROUP_WORKSPACE_BYTES} bytes")
    _check("sp24_spmm_group", lib().sp24_spmm_group(ctypes.cast(descs, ctypes.c_void_p), len(gemms), _ptr(ws),
                                                    _stream(stream)))
    return outs
