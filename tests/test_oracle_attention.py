"""Pins of the attention oracle against closed forms, a library routine and brute force."""
import numpy as np
import pytest

import pins
from oracle import attention as A
from oracle import layout
from oracle.numerics import to_f64
from workloads import bf16_bits_from_f32


@pytest.mark.parametrize("check", pins.ATTN_CHECKS, ids=lambda f: f.__name__)
def test_attention_pins(check):
    check(A.softmax_attention)


def test_probs_sum_to_one():
    pins.check_probs_sum_to_one(lambda k, v, q, s: A.softmax_attention(k, v, q, s, return_probs=True))


def test_verify_causal():
    pins.check_verify_causal(A.verify, A.softmax_attention)


def test_empty_context_rejected():
    with pytest.raises(ValueError):
        A.softmax_attention(np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), np.zeros((1, 4)), 1.0)


def test_numerics_decode_exact():
    x = np.array([1.0, -2.5, 3.140625, 65504.0, 2.0 ** -24], dtype=np.float32)
    assert np.array_equal(to_f64(x, "f32"), x.astype(np.float64))
    h = x.astype(np.float16)
    assert np.array_equal(to_f64(h, "f16"), h.astype(np.float64))
    b = bf16_bits_from_f32(np.array([1.0, -2.5, 3.140625, 1.00390625, 1.01171875], np.float32))
    # 1.00390625 = 1 + 2^-8 is a tie between 1 and 1 + 2^-7 in bf16 -> even (1.0);
    # 1.01171875 = 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
    assert np.array_equal(to_f64(b, "bf16"), [1.0, -2.5, 3.140625, 1.0, 1.015625])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_layout_offsets_match_arrays(dtype):
    """The flat-offset formula and the shaped-array view name the same element."""
    nb, hkv, d = 3, 2, 32
    kshape = layout.k_shape(nb, hkv, d, dtype)
    vshape = layout.v_shape(nb, hkv, d, dtype)
    kflat = np.arange(np.prod(kshape))
    vflat = np.arange(np.prod(vshape))
    k5 = kflat.reshape(kshape)
    v4 = vflat.reshape(vshape)
    r = np.random.default_rng(0)
    for _ in range(200):
        b, h, t, j = r.integers(nb), r.integers(hkv), r.integers(16), r.integers(d)
        krow, vrow = layout.read_row(k5, v4, b, t, dtype)
        assert krow[h, j] == layout.k_offset(b, h, t, j, hkv, d, dtype)
        assert vrow[h, j] == layout.v_offset(b, h, t, j, hkv, d)
    # every element is reachable exactly once
    seen = {layout.k_offset(b, h, t, j, hkv, d, dtype)
            for b in range(nb) for h in range(hkv) for t in range(16) for j in range(d)}
    assert seen == set(range(int(np.prod(kshape))))


def test_gather_through_table_equals_contiguous():
    """Rows written at scattered blocks and read back through the table give the
    contiguous rows ([P2] section 4.1: blocks treated as if contiguous)."""
    r = np.random.default_rng(3)
    nb, hkv, d, n = 10, 2, 8, 37
    k5 = np.zeros(layout.k_shape(nb, hkv, d, "f32"), np.float32)
    v4 = np.zeros(layout.v_shape(nb, hkv, d, "f32"), np.float32)
    table = [7, 2, 9]
    rows_k = r.standard_normal((n, hkv, d)).astype(np.float32)
    rows_v = r.standard_normal((n, hkv, d)).astype(np.float32)
    for t in range(n):
        layout.write_row(k5, v4, table[t // 16], t % 16, rows_k[t], rows_v[t], "f32")
    kc, vc = A.gather(k5, v4, table, n, "f32")
    assert np.array_equal(kc, rows_k.astype(np.float64))
    assert np.array_equal(vc, rows_v.astype(np.float64))
