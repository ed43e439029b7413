"""Pins of the byte accounting against the figures the pages print
(tests/golden/pages_figures.json, each entry citing its page and section)."""
import json
import math
import os

import pytest

from oracle import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_bandwidth_wall_example():
    g = GOLDEN["bandwidth_wall"]
    weights = g["params"] * g["bytes_per_param"]
    assert weights == pytest.approx(g["weights_gb"] * 1e9)
    t = acc.bandwidth_bound_time(weights, g["bandwidth_gb_s"] * 1e9)
    assert t == pytest.approx(g["seconds_per_token"])
    assert round(1.0 / t) == g["tokens_per_second_approx"]


def test_contiguous_reservation_example():
    g = GOLDEN["contiguous_reservation"]
    assert acc.contiguous_unused(g["used_tokens"], g["reserved_tokens"]) > g["unused_fraction_greater_than"]


def test_paged_waste_example():
    g = GOLDEN["paged_waste"]
    n = g["example_length"]
    waste = acc.paged_unused_slots(n, GOLDEN["block_size"]["tokens_per_block"])
    assert waste == 8                    # 200 tokens -> 13 blocks -> 208 slots
    assert waste / (n + waste) < g["max_unused_fraction"]
    assert all(acc.paged_unused_slots(k) <= 15 for k in range(1, 500))


def test_kv_formula_terms():
    """Each of the seven factors enters linearly (double one, the size doubles)."""
    base = dict(batch=3, seq_len=100, layers=2, heads=8, head_dim=128, bytes_per_value=2)
    b0 = acc.kv_cache_bytes(**base)
    assert b0 == 2 * 3 * 100 * 2 * 8 * 128 * 2
    for k in base:
        d = dict(base)
        d[k] *= 2
        assert acc.kv_cache_bytes(**d) == 2 * b0


def test_decode_step_bytes_matches_kv_formula():
    """One decode step reads the whole cache ([P3] section 3 table): with equal
    lengths, the K/V part equals the section-3.2 formula for one layer."""
    b, n, hkv, hq, d, e = 4, 64, 8, 32, 128, 2
    tot = acc.decode_step_bytes([n] * b, hkv, hq, d, e)
    kv = acc.kv_cache_bytes(b, n, 1, hkv, d, e)
    assert tot == kv + 2 * b * hq * d * e + b * math.ceil(n / 16) * 4 + 4 * b
    # a shared prefix is counted once
    shared = acc.decode_step_bytes([n + 16] * b, hkv, hq, d, e, shared_prefix_tokens=n)
    assert shared == (n + 16 * b) * hkv * d * e * 2 + 2 * b * hq * d * e + b * 5 * 4 + 4 * b
