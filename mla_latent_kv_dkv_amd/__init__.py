"""MLA latent-KV decode for MI355X (gfx950): Python binding over libmla.so.

The compute lives in hand-written HIP kernels behind a C ABI; this package only
marshals arguments.  The native library is loaded on first use and its absence
is an error (there is no CPU fallback).
"""
