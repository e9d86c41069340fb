"""The compressed 2:4 forms' blocked order, as the C header defines it.

The library stores each logical n x m matrix of a form (vals: m = C/2 halves
per row, block width 32; meta: m = C/16 words per row, block width 4) as bands
of 64 rows (the last band may be shorter); a band holds its column blocks one
after the other (the last block of a row may be narrower), each block
row-major.  The oracle writes the forms row-major, as the method defines them.
Tests put the oracle's forms into the blocked order before handing them to the
library, and take the library's forms back out of it before comparing.  This is
a pure permutation, built here band by band and block by block from that
definition; nothing in it computes any part of the method.
"""
from functools import lru_cache

import numpy as np

VALS_BLOCK, META_BLOCK = 32, 4
BAND = 64


def block_width(key: str) -> int:
    return META_BLOCK if key.startswith("meta") else VALS_BLOCK


@lru_cache(maxsize=8)
def _positions(n: int, m: int, b: int) -> np.ndarray:
    pos = np.empty((n, m), np.int64)
    at = 0
    for r0 in range(0, n, BAND):
        h = min(BAND, n - r0)
        for c0 in range(0, m, b):
            w = min(b, m - c0)
            pos[r0:r0 + h, c0:c0 + w] = at + np.arange(h * w).reshape(h, w)
            at += h * w
    assert at == n * m
    pos.setflags(write=False)
    return pos


def blocked_positions(n: int, m: int, b: int) -> np.ndarray:
    """pos[r, c]: where element (r, c) of a row-major n x m matrix sits in the blocked order."""
    return _positions(int(n), int(m), int(b))


def to_blocked(a: np.ndarray, b: int) -> np.ndarray:
    """The row-major matrix a in blocked order (returned with a's 2-D shape)."""
    a = np.ascontiguousarray(a)
    n, m = a.shape
    out = np.empty(n * m, a.dtype)
    out[blocked_positions(n, m, b).ravel()] = a.ravel()
    return out.reshape(n, m)


def from_blocked(a: np.ndarray, b: int) -> np.ndarray:
    """The row-major matrix whose blocked order is a (a has the logical 2-D shape)."""
    n, m = a.shape
    return np.ascontiguousarray(a).reshape(-1)[blocked_positions(n, m, b)]


def forms_to_blocked(forms: dict) -> dict:
    """Copy of a dict of forms with every vals_* / meta_* entry in blocked order."""
    return {k: (to_blocked(v, block_width(k)) if k.startswith(("vals", "meta")) else v) for k, v in forms.items()}
