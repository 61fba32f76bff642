"""Exact tiled attention (online softmax) for AMD MI355X (gfx950).

The compute lives in a C-ABI HIP shared library (libfa_gfx950.so, built from
csrc/); `fa` is a thin ctypes binding over it with the same entry-point names.
The library is loaded on first use and the binding raises if it is missing:
there is no CPU fallback.
"""
