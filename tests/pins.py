"""Pin checks for the attention oracle.

Each ``check_*`` takes the attention functions under test (by default the
oracle's) and raises AssertionError when the pinned property fails.  The pin
tests call them on the oracle; the planted-mistake tests call them on mutated
copies and expect at least one check to fail.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def check_single_token(attn):
    """One cached row: the softmax weight is exactly 1, so O is that V row and
    lse is the scaled score."""
    r = _rng(10)
    kc = r.standard_normal((1, 2, 8))
    vc = r.standard_normal((1, 2, 8))
    q = r.standard_normal((4, 8))
    o, lse = attn(kc, vc, q, 0.3)[:2]
    for h in range(4):
        kvh = h // 2
        assert np.array_equal(o[h], vc[0, kvh]), "single token must return its V row exactly"
        assert abs(lse[h] - 0.3 * float(q[h] @ kc[0, kvh])) < 1e-12


def check_identical_keys(attn):
    """All keys equal: uniform weights, O = mean of V, lse = x + ln n."""
    r = _rng(11)
    n = 37
    k = r.standard_normal(16)
    kc = np.broadcast_to(k, (n, 1, 16)).copy()
    vc = r.standard_normal((n, 1, 16))
    q = r.standard_normal((3, 16))
    o, lse = attn(kc, vc, q, 0.25)[:2]
    for h in range(3):
        assert np.allclose(o[h], vc[:, 0].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[h] - (0.25 * float(q[h] @ k) + math.log(n))) < 1e-12


def check_constant_values(attn):
    """Every V row equal to c: O = c whatever the weights."""
    r = _rng(12)
    n = 50
    kc = r.standard_normal((n, 2, 8)) * 3
    c = r.standard_normal((2, 8))
    vc = np.broadcast_to(c, (n, 2, 8)).copy()
    q = r.standard_normal((6, 8))
    o = attn(kc, vc, q, 0.5)[0]
    for h in range(6):
        assert np.allclose(o[h], c[h // 3], atol=1e-13, rtol=0)


def check_zero_scale(attn):
    """scale = 0: uniform weights whatever the keys; lse = ln n."""
    r = _rng(13)
    n = 23
    kc = r.standard_normal((n, 2, 8))
    vc = r.standard_normal((n, 2, 8))
    q = r.standard_normal((2, 8))
    o, lse = attn(kc, vc, q, 0.0)[:2]
    for h in range(2):
        assert np.allclose(o[h], vc[:, h].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[h] - math.log(n)) < 1e-12


def check_probs_sum_to_one(attn_probs):
    r = _rng(14)
    kc = r.standard_normal((100, 2, 16)) * 4
    vc = r.standard_normal((100, 2, 16))
    q = r.standard_normal((8, 16))
    _, _, p = attn_probs(kc, vc, q, 0.7)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12


def torch_sdpa_reference(kc, vc, q, scale, mask=None):
    """Library routine on contiguous rows: K/V repeated per query-head group."""
    n, hkv, d = kc.shape
    hq = q.shape[-2]
    g = hq // hkv
    kt = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(g, dim=0)  # [Hq, n, D]
    vt = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(g, dim=0)
    if q.ndim == 2:
        qt = torch.from_numpy(q)[:, None, :]           # [Hq, 1, D]
    else:
        qt = torch.from_numpy(q).permute(1, 0, 2)      # [Hq, K, D]
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.contiguous(), kt.contiguous(), vt.contiguous(), attn_mask=am, scale=scale)
    if q.ndim == 2:
        return o[:, 0, :].numpy()
    return o.permute(1, 0, 2).numpy()


def check_against_sdpa(attn):
    r = _rng(15)
    for n, hkv, g, d in [(1, 1, 1, 8), (17, 2, 4, 32), (100, 4, 1, 64), (257, 2, 8, 16)]:
        kc = r.standard_normal((n, hkv, d))
        vc = r.standard_normal((n, hkv, d))
        q = r.standard_normal((hkv * g, d))
        s = 1.0 / math.sqrt(d)
        o = attn(kc, vc, q, s)[0]
        ref = torch_sdpa_reference(kc, vc, q, s)
        assert np.allclose(o, ref, atol=1e-12, rtol=1e-12), (n, hkv, g, d)


def naive_attention(kc, vc, q, scale):
    """Triple loop in pure Python, contiguous query-head groups."""
    n, hkv, d = kc.shape
    hq = q.shape[0]
    g = hq // hkv
    out = [[0.0] * d for _ in range(hq)]
    lse = [0.0] * hq
    for h in range(hq):
        kvh = h // g
        xs = []
        for t in range(n):
            acc = 0.0
            for j in range(d):
                acc += float(q[h, j]) * float(kc[t, kvh, j])
            xs.append(scale * acc)
        m = max(xs)
        es = [math.exp(x - m) for x in xs]
        z = sum(es)
        for j in range(d):
            out[h][j] = sum(es[t] / z * float(vc[t, kvh, j]) for t in range(n))
        lse[h] = m + math.log(z)
    return np.array(out), np.array(lse)


def check_against_naive(attn):
    r = _rng(16)
    kc = r.standard_normal((9, 2, 4))
    vc = r.standard_normal((9, 2, 4))
    q = r.standard_normal((4, 4))
    o, lse = attn(kc, vc, q, 0.9)[:2]
    o2, lse2 = naive_attention(kc, vc, q, 0.9)
    assert np.allclose(o, o2, atol=1e-13, rtol=0)
    assert np.allclose(lse, lse2, atol=1e-13, rtol=0)


def check_gqa_grouping(attn):
    """G copies of one query in a group give G equal outputs; different KV heads
    give different outputs; G = 1 is per-head attention."""
    r = _rng(17)
    kc = r.standard_normal((40, 4, 8))
    vc = r.standard_normal((40, 4, 8))
    base = r.standard_normal((4, 8))
    q = np.repeat(base, 3, axis=0)  # heads 0,1,2 share base[0], ...
    o = attn(kc, vc, q, 0.4)[0]
    for kvh in range(4):
        for g in range(3):
            assert np.array_equal(o[kvh * 3 + g], o[kvh * 3])
        ref = attn(kc[:, kvh:kvh + 1], vc[:, kvh:kvh + 1], base[kvh:kvh + 1], 0.4)[0][0]
        assert np.allclose(o[kvh * 3], ref, atol=1e-14, rtol=0)


def check_lse_merge(attn):
    """Attention over a split context, recombined with the returned lse, equals
    attention over the whole context (the identity a split-context kernel uses)."""
    r = _rng(18)
    kc = r.standard_normal((70, 2, 8)) * 2
    vc = r.standard_normal((70, 2, 8))
    q = r.standard_normal((4, 8))
    o, lse = attn(kc, vc, q, 0.6)[:2]
    parts = [(0, 13), (13, 50), (50, 70)]
    res = [attn(kc[a:b], vc[a:b], q, 0.6)[:2] for a, b in parts]
    big = np.max(np.stack([l_ for _, l_ in res]), axis=0)
    w = np.stack([np.exp(l_ - big) for _, l_ in res])         # [P, Hq]
    merged = sum(w[i][:, None] * res[i][0] for i in range(len(parts))) / w.sum(axis=0)[:, None]
    assert np.allclose(merged, o, atol=1e-13, rtol=0)
    assert np.allclose(big + np.log(w.sum(axis=0)), lse, atol=1e-13, rtol=0)


def check_verify_causal(verify, attn):
    """Draft i of K attends to rows [0, n-K+i]: it equals a decode of the
    sequence cut at n-K+i+1, and a masked library attention."""
    r = _rng(19)
    n, kd = 30, 5
    kc = r.standard_normal((n, 2, 8))
    vc = r.standard_normal((n, 2, 8))
    q = r.standard_normal((kd, 4, 8))
    o, lse = verify(kc, vc, q, 0.5)
    for i in range(kd):
        oi, li = attn(kc[:n - kd + i + 1], vc[:n - kd + i + 1], q[i], 0.5)[:2]
        assert np.array_equal(o[i], oi)
        assert np.array_equal(lse[i], li)
    mask = np.zeros((kd, n), dtype=bool)
    for i in range(kd):
        mask[i, : n - kd + i + 1] = True
    ref = torch_sdpa_reference(kc, vc, q, 0.5, mask=mask)
    assert np.allclose(o, ref, atol=1e-12, rtol=1e-12)
    # a draft must see its own row: with K=1 verify is a plain decode
    o1, _ = verify(kc, vc, q[:1], 0.5)
    assert np.array_equal(o1[0], attn(kc, vc, q[0], 0.5)[0])


ATTN_CHECKS = [
    check_single_token, check_identical_keys, check_constant_values, check_zero_scale,
    check_against_sdpa, check_against_naive, check_gqa_grouping, check_lse_merge,
]
