"""Hybrid Top-k + Top-p block-sparse attention on MI355X (gfx950).

The compute lives in ``libsparge.so`` (hand-written HIP kernels behind a C
ABI). This package is a thin ctypes binding over it; importing the binding
loads the library and fails loudly if it has not been built.
"""
