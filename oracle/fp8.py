"""8-bit floating point KV-cache codes (E4M3, the OCP "fn" variant) -- test
infrastructure, part of the CPU oracle.

Storing the key/value cache in 8 bits halves the bytes a decode step reads,
with the softmax and the accumulation kept at full precision (ranksignal.fr
post 218, "Quantifier", which names FP8 and INT8 caches).  The pages fix no
format; this library's reading is E4M3 with one scale per (key or value,
KV head): stored code c for input x is E4M3(x * inv_scale), and the value
the attention uses is decode(c) * scale.

E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field
0 holds the subnormals m * 2**-9; exponent e in 1..15 holds (1 + m/8) * 2**(e-7)
except e = 15, m = 7, which is NaN.  There is no infinity; the largest finite
magnitude is 448.  Encoding clamps to [-448, 448] and then rounds to the
nearest code, ties to the even code (even mantissa).

The encoder below is written from that definition by brute force: the
nearest of the 127 non-negative finite values (compared all at once, a chunk
of inputs at a time), so that it can be checked by eye.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode_code(c: int) -> float:
    """Value of one E4M3 code (0..255), NaN for the two NaN codes."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
_POS = TABLE[:0x7F]  # codes 0x00 .. 0x7E: 0 and the positive finite values, ascending


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of codes (uint8)."""
    return TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """Codes (uint8) of float32 values: clamp to +-448, round to nearest, ties
    to the even code.  The sign of the input is kept, zero included."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1).astype(np.float64)
    out = np.empty(flat.shape, dtype=np.uint8)
    even = (np.arange(_POS.size) % 2 == 0)
    for lo in range(0, flat.size, 1 << 15):
        v = flat[lo:lo + (1 << 15)]
        a = np.minimum(np.abs(v), MAX_FINITE)
        # distance of every input to every candidate value; the nearest wins,
        # and between two equally near candidates the even code
        d = np.abs(_POS[None, :] - a[:, None])
        best = d.min(axis=1, keepdims=True)
        tie_ok = (d == best) & (even[None, :] | ((d == best).sum(axis=1, keepdims=True) == 1))
        code = np.argmax(tie_ok, axis=1).astype(np.uint8)
        code |= np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
        code[np.isnan(v)] = 0x7F
        out[lo:lo + v.size] = code
    return out.reshape(x.shape)


def encode_by_search(x: np.ndarray) -> np.ndarray:
    """The same codes as ``encode``, found by a binary search of the sorted
    non-negative values instead of comparing against all of them: after the
    clamp, the nearest value is one of the two around the input; an input
    exactly between them takes the even code.  For bulk inputs (whole
    full-size caches); tests check it equals ``encode`` on every bf16 value,
    every midpoint between neighbouring codes and random float32 inputs."""
    x = np.asarray(x, dtype=np.float32)
    v = x.reshape(-1).astype(np.float64)
    a = np.minimum(np.abs(v), MAX_FINITE)
    hi = np.minimum(np.searchsorted(_POS, a, side="left"), _POS.size - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    code = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    code = code.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    code[np.isnan(v)] = 0x7F
    return code.reshape(x.shape)
