"""Decode stored element bit patterns to float64 (oracle; test infrastructure only).

Storage types: 'f32' (IEEE binary32), 'f16' (IEEE binary16), 'bf16' (the top
16 bits of a binary32), 'fp8' (E4M3 codes, oracle/fp8.py; decoded unscaled).
Arrays arrive either as float32/float16 numpy arrays or as raw unsigned bit
patterns (uint32 / uint16 / uint8); all decode exactly.
"""
from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


def as_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """View a storage array as its raw bit patterns."""
    a = np.ascontiguousarray(a)
    want = BITS_DTYPE[dtype]
    if a.dtype == want:
        return a
    if a.dtype.itemsize != np.dtype(want).itemsize:
        raise TypeError(f"{a.dtype} is not a {dtype} storage array")
    return a.view(want)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every stored element."""
    bits = as_bits(a, dtype)
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        from .fp8 import decode
        return decode(bits)
    raise ValueError(dtype)
