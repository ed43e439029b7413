"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

libpa.so (C ABI in include/pa.h) holds the block allocator and the HIP kernels;
this package is a thin binding over it.  Build it first:

    python -m paged_kv_cache_216_amd.build
"""
from . import abi  # noqa: F401
from .abi import PaError, PaHipError, PaInvalid, PaNoMem, PaStateError  # noqa: F401


def __getattr__(name):
    # import the torch-based binding lazily so that `abi` can be used without torch
    if name in ("PagedKVCache", "cache"):
        from . import cache
        return cache if name == "cache" else cache.PagedKVCache
    raise AttributeError(name)
