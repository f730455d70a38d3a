"""Paged-KV attention for AMD MI355X (gfx950): Python binding of libpkv.

The library (HIP kernels behind a C ABI, ``include/pkv.h``) is loaded on first
use from this directory.
"""
