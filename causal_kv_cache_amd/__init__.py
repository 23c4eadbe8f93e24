"""Shared causal KV-cache attention for autoregressive video diffusion on MI355X.

The computation lives in libca2.so (HIP kernels for gfx950 behind the C ABI of
include/ca2.h); ``causal_kv_cache_amd.ca2`` is its ctypes binding. Importing
the package loads nothing; ``ca2.load()`` does, and fails if the library has
not been built.
"""
__all__ = ["ca2"]
