"""Transposable 2:4 sparse FFN kernels for MI355X (gfx950).

The compute lives in ``libsp24.so`` (HIP kernels behind the C ABI of
``include/sp24.h``); :mod:`structured_sparse_transformer_amd.sp24` is the thin
ctypes binding.  Build the library with
``python -m structured_sparse_transformer_amd.build``.
"""
