"""Pins for the oracle's E4M3 codes (oracle/fp8.py): closed-form values of
the format's definition, round trips, the tie rule, saturation and the
rounding error bound."""
import math

import numpy as np
import pytest

from oracle import fp8


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x30, 0.5),
    (0x7E, 448.0), (0x77, 240.0), (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9), (0x01, 2.0 ** -9),
    (0xB8, -1.0), (0xFE, -448.0),
])
def test_decode_closed_forms(code, value):
    assert fp8.decode_code(code) == value


def test_nan_codes_and_signed_zero():
    assert math.isnan(fp8.decode_code(0x7F)) and math.isnan(fp8.decode_code(0xFF))
    assert fp8.decode_code(0x80) == 0.0 and math.copysign(1.0, fp8.decode_code(0x80)) == -1.0
    assert fp8.encode(np.array([-0.0], np.float32))[0] == 0x80
    assert fp8.encode(np.array([0.0], np.float32))[0] == 0x00


def test_positive_values_strictly_increase():
    v = fp8.TABLE[:0x7F]
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(fp8.TABLE[0x80:0xFF], -v)


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes).astype(np.float32)), codes)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),        # halfway 1.0 / 1.125: even mantissa (1.0)
    (1.1875, 0x3A),        # halfway 1.125 / 1.25: even mantissa (1.25)
    (2.0 ** -10, 0x00),    # halfway 0 / smallest subnormal
    (1.5 * 2.0 ** -9, 0x02),
    (-1.0625, 0xB8),
    (1.07, 0x39), (1.06, 0x38), (1.0624, 0x38),
])
def test_ties_to_even_and_nearest(x, code):
    assert fp8.encode(np.array([x], np.float32))[0] == code


@pytest.mark.parametrize("x,code", [(448.0, 0x7E), (460.0, 0x7E), (500.0, 0x7E), (1e30, 0x7E), (-1e6, 0xFE)])
def test_saturation(x, code):
    assert fp8.encode(np.array([x], np.float32))[0] == code


def test_error_within_half_spacing():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4000) * rng.choice([1e-3, 1.0, 30.0], 4000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    y = fp8.decode(fp8.encode(x))
    a = np.abs(x.astype(np.float64))
    # spacing of the format at |x|: 2**-9 in the subnormal range, else 2**(floor(log2|x|) - 3)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
    assert np.all(np.abs(y - x) <= spacing / 2 + 1e-12)


def test_planted_tie_rule_is_caught():
    """Rounding ties away from zero (a plausible slip) breaks the tie pins."""
    x = np.float32(1.0625)
    away = 0x39  # 1.125
    assert fp8.encode(np.array([x]))[0] != away


def test_pool_model_stores_scaled_codes_and_gather_rescales():
    """An 'fp8' pool model stores E4M3(x / scale[h]) per kv head and its gather
    returns decode(code) * scale[h]: 1.0 at scale 0.5 is code 0x40 (2.0),
    -3.0 at scale 2.0 is 0xBC (-1.5), 1000 at scale 1 saturates to 0x7E."""
    from oracle import attention as A
    from oracle.allocator import PoolModel

    def bf16(a):
        return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    m = PoolModel(4, 3, 64, "fp8", 2, 2, kv_scales=(np.array([0.5, 2.0, 1.0], np.float32),
                                                    np.array([1.0, 1.0, 4.0], np.float32)))
    m.alloc(0)
    k = np.zeros((1, 3, 64), np.float32)
    v = np.zeros((1, 3, 64), np.float32)
    k[0, 0, :] = 1.0
    k[0, 1, :] = -3.0
    k[0, 2, :] = 1000.0
    v[0, 2, :] = 6.0  # 6 / 4 = 1.5 -> 0x3C
    m.append([0], [1], bf16(k), bf16(v))
    kc, vc = A.gather(m.kpool, m.vpool, m.table(0), 1, "fp8")
    assert np.all(kc[0, 0] == 2.0) and np.all(kc[0, 1] == -1.5) and np.all(kc[0, 2] == 448.0)
    assert np.all(vc[0, 2] == 1.5) and np.all(vc[0, :2] == 0.0)
    ks, vs = A.gather(m.kpool, m.vpool, m.table(0), 1, "fp8", (m.k_scale, m.v_scale))
    assert np.all(ks[0, 0] == 1.0) and np.all(ks[0, 1] == -3.0) and np.all(ks[0, 2] == 448.0)
    assert np.all(vs[0, 2] == 6.0)


def test_search_encoder_equals_brute_force():
    """encode_by_search gives the brute-force encoder's code for every finite
    bf16 value, every midpoint between neighbouring codes (and a float32 ulp
    either side), values past the clamp and random float32 inputs."""
    from oracle.fp8 import _POS, encode_by_search

    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    mids = ((_POS[1:] + _POS[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rnd = np.random.default_rng(5).standard_normal(200_000).astype(np.float32) * np.float32(40)
    for arr in (x, near, -near, rnd, np.array([448.0, 449.0, 464.0, 1e30, -1e30, 0.0, -0.0], np.float32)):
        assert np.array_equal(encode_by_search(arr), fp8.encode(arr))
