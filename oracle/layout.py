"""Physical pool layout contract, written out plainly (oracle; test infrastructure only).

The pages fix only that the cache is cut into fixed blocks of 16 tokens that may
sit anywhere in memory, reached through a block table ([P1] section 1; [P2]
section 4.1).  The byte layout inside a block is this library's contract:

  K pool: [num_blocks][num_kv_heads][head_dim / X][16][X]   X = 16 bytes / element size
  V pool: [num_blocks][num_kv_heads][head_dim][16]

i.e. element d of token slot t of (block b, head h) is stored at
  K: ((((b * Hkv + h) * (D / X) + d // X) * 16 + t) * X + d % X
  V: (((b * Hkv + h) * D + d) * 16 + t
"""
from __future__ import annotations

import numpy as np

from .numerics import ELEM_BYTES

BLOCK = 16


def chunk(dtype: str) -> int:
    return 16 // ELEM_BYTES[dtype]


def k_shape(num_blocks: int, hkv: int, d: int, dtype: str):
    x = chunk(dtype)
    assert d % x == 0
    return (num_blocks, hkv, d // x, BLOCK, x)


def v_shape(num_blocks: int, hkv: int, d: int, dtype: str):
    return (num_blocks, hkv, d, BLOCK)


def k_offset(b: int, h: int, t: int, d: int, hkv: int, head_dim: int, dtype: str) -> int:
    """Flat element offset of K[b, h, slot t, dim d] (the formula in the docstring)."""
    x = chunk(dtype)
    return ((((b * hkv + h) * (head_dim // x) + d // x) * BLOCK + t) * x) + d % x


def v_offset(b: int, h: int, t: int, d: int, hkv: int, head_dim: int) -> int:
    return ((b * hkv + h) * head_dim + d) * BLOCK + t


def write_row(kpool: np.ndarray, vpool: np.ndarray, b: int, t: int,
              k_row: np.ndarray, v_row: np.ndarray, dtype: str) -> None:
    """Store one token's K and V rows ([Hkv, D] each) at slot t of block b.

    ``kpool`` / ``vpool`` are the 5-d / 4-d arrays of ``k_shape`` / ``v_shape``.
    """
    hkv, d = k_row.shape
    x = chunk(dtype)
    kpool[b, :, :, t, :] = k_row.reshape(hkv, d // x, x)
    vpool[b, :, :, t] = v_row


def read_row(kpool: np.ndarray, vpool: np.ndarray, b: int, t: int, dtype: str):
    """Inverse of ``write_row``: the [Hkv, D] K and V rows at slot t of block b."""
    hkv = kpool.shape[1]
    k = kpool[b, :, :, t, :].reshape(hkv, -1)
    v = vpool[b, :, :, t]
    return k.copy(), v.copy()


def copy_rows(kpool: np.ndarray, vpool: np.ndarray, src: int, dst: int, n_rows: int) -> None:
    """Copy slots [0, n_rows) of every head from block src to block dst."""
    kpool[dst, :, :, :n_rows, :] = kpool[src, :, :, :n_rows, :]
    vpool[dst, :, :, :n_rows] = vpool[src, :, :, :n_rows]
