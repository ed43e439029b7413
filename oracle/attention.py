"""Reference attention over a paged KV cache, in float64 (oracle; test infrastructure only).

Definition followed.  The cache keeps the K and V rows of every past token so
that the new token's query only has to attend over them ([P1] section 1; [P2]
section 3.1 and its data-flow graph: K(t), V(t) are stored, then the past cache
and Q(t) feed the attention).  Paging changes where the rows live, not the
result: the blocks are treated as if they were contiguous ([P2] section 4.1), the
table being resolved inside the attention ([P1] section 1).  So the reference is:

  1. gather the sequence's rows through its block table into contiguous arrays;
  2. ordinary softmax attention for each query head h, with key/value head
     kvh = h // (Hq / Hkv) (contiguous query-head groups):
        x_t   = scale * sum_d q[h, d] * K[t, kvh, d]
        m     = max_t x_t
        p_t   = exp(x_t - m) / sum_u exp(x_u - m)
        O[h]  = sum_t p_t * V[t, kvh, :]
        lse   = m + ln sum_u exp(x_u - m)
     The score and probability matrices never need to be stored by a fused
     kernel ([P4] "Les noyaux d'attention"); here they are plain arrays.

Speculative verify ([P1] section 1; [P2] section 5.2; [P4] "Spéculer"): the K
draft tokens were appended to the cache, and draft i (0-based) attends to every
token up to and including itself, i.e. to positions [0, L + i] where L is the
length before the drafts.  Its result therefore equals a plain decode of the
sequence cut at L + i + 1 tokens, which is how it is computed below.
"""
from __future__ import annotations

import numpy as np

from . import layout
from .numerics import to_f64

BLOCK = layout.BLOCK


def gather(kpool: np.ndarray, vpool: np.ndarray, block_table, n: int, dtype: str, kv_scales=None):
    """Rows 0..n-1 of one sequence as float64 arrays [n, Hkv, D].

    ``kpool`` / ``vpool`` are the 5-d / 4-d pool arrays of ``oracle.layout``
    (bit patterns or float arrays of the storage type).  For 'fp8' pools,
    ``kv_scales`` = (k_scale[Hkv], v_scale[Hkv]) multiply the decoded codes.
    """
    hkv = kpool.shape[1]
    d = vpool.shape[2]
    kc = np.empty((n, hkv, d), dtype=np.float64)
    vc = np.empty((n, hkv, d), dtype=np.float64)
    for t in range(n):
        b = int(block_table[t // BLOCK])
        k, v = layout.read_row(kpool, vpool, b, t % BLOCK, dtype)
        kc[t] = to_f64(k, dtype)
        vc[t] = to_f64(v, dtype)
    if kv_scales is not None:
        kc *= np.asarray(kv_scales[0], np.float64)[None, :, None]
        vc *= np.asarray(kv_scales[1], np.float64)[None, :, None]
    return kc, vc


def softmax_attention(kc: np.ndarray, vc: np.ndarray, q: np.ndarray, scale: float,
                      return_probs: bool = False):
    """Decode attention of one query token over contiguous float64 rows.

    kc, vc: [n, Hkv, D]; q: [Hq, D] (float64).  Returns O [Hq, D], lse [Hq] and,
    if asked, the probabilities [Hq, n].
    """
    n, hkv, d = kc.shape
    hq = q.shape[0]
    if n == 0:
        raise ValueError("attention over an empty context is undefined")
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    g = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    lse = np.empty(hq, dtype=np.float64)
    probs = np.empty((hq, n), dtype=np.float64)
    for h in range(hq):
        kvh = h // g
        x = scale * (kc[:, kvh, :] @ q[h])
        m = np.max(x)
        e = np.exp(x - m)
        s = np.sum(e)
        p = e / s
        out[h] = p @ vc[:, kvh, :]
        lse[h] = m + np.log(s)
        probs[h] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def decode(kc: np.ndarray, vc: np.ndarray, q: np.ndarray, scale: float):
    """One query per sequence over all n cached rows (O [Hq, D], lse [Hq])."""
    return softmax_attention(kc, vc, q, scale)


def verify(kc: np.ndarray, vc: np.ndarray, q: np.ndarray, scale: float):
    """K draft queries q [K, Hq, D] over n rows whose last K are the drafts.

    Draft i sees rows [0, n - K + i]; returns O [K, Hq, D], lse [K, Hq].
    """
    n = kc.shape[0]
    kd = q.shape[0]
    if n < kd:
        raise ValueError("the drafts must already be in the cache")
    outs, lses = [], []
    for i in range(kd):
        ni = n - kd + i + 1
        o, l_ = softmax_attention(kc[:ni], vc[:ni], q[i], scale)
        outs.append(o)
        lses.append(l_)
    return np.stack(outs), np.stack(lses)


def decode_from_pool(kpool, vpool, block_table, n: int, q_bits: np.ndarray, scale: float,
                     dtype: str, kv_scales=None):
    """Gather + decode for one sequence; q_bits [Hq, D] in the storage type."""
    kc, vc = gather(kpool, vpool, block_table, n, dtype, kv_scales)
    return decode(kc, vc, to_f64(q_bits, "bf16" if dtype == "fp8" else dtype), scale)


def verify_from_pool(kpool, vpool, block_table, n: int, q_bits: np.ndarray, scale: float,
                     dtype: str, kv_scales=None):
    """Gather + verify for one sequence; q_bits [K, Hq, D] in the storage type."""
    kc, vc = gather(kpool, vpool, block_table, n, dtype, kv_scales)
    return verify(kc, vc, to_f64(q_bits, "bf16" if dtype == "fp8" else dtype), scale)
