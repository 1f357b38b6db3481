"""Streaming block-causal chunk attention on AMD MI355X (gfx950).

The compute lives in libswattn.so (HIP kernels + C ABI, include/swattn.h);
`native` is its ctypes binding with the C names, `cache.Cache` a torch-facing
wrapper that owns the device pool.  Build with
`python -m streaming_block_causal_amd.build`.
"""
from .native import SwError, lib  # noqa: F401


def __getattr__(name):
    if name in ("Cache", "CacheConfig"):
        from . import cache
        return getattr(cache, name)
    raise AttributeError(name)
