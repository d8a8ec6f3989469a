"""Pins of the oracle's scalar numerics: bf16 rounding and MXFP4 decoding.

bf16 rounding is pinned by hand-derived tie cases and by a nearest-value search
over the table of all bf16 values (a different method). e2m1 is pinned by the
OCP MX v1.0 value table written out in tests/golden; e8m0 by its closed form at
chosen bytes; the nibble order and scale-block index by one-hot rows."""

import math

import numpy as np
import pytest

import oracle
from tests._ref import e2m1_table, nearest_bf16_bits


def test_bf16_to_f64_known_bits():
    assert oracle.bf16_to_f64(0x3F80) == 1.0
    assert oracle.bf16_to_f64(0xC000) == -2.0
    assert oracle.bf16_to_f64(0x3FC0) == 1.5
    assert oracle.bf16_to_f64(0x0001) == 2.0**-133
    assert oracle.bf16_to_f64(0x7F7F) == (2 - 2**-7) * 2.0**127
    assert math.isinf(oracle.bf16_to_f64(0x7F80))
    v = oracle.bf16_to_f64(0x8000)
    assert v == 0.0 and math.copysign(1, v) < 0


@pytest.mark.parametrize(
    "v,bits",
    [
        (1.0, 0x3F80),
        (1 + 2**-8, 0x3F80),  # halfway 1 .. 1+2^-7: to the even significand (1)
        (1 + 2**-8 + 2**-30, 0x3F81),  # just above halfway
        (1 + 3 * 2**-8, 0x3F82),  # halfway 1+2^-7 .. 1+2^-6: to even (..82)
        (1 + 3 * 2**-8 - 2**-30, 0x3F81),
        (-(1 + 2**-8), 0xBF80),
        ((2 - 2**-7) * 2.0**127, 0x7F7F),  # largest finite
        ((2 - 2**-7) * 2.0**127 + 2.0**119, 0x7F80),  # tie at the top: to even = inf
        ((2 - 2**-7) * 2.0**127 + 2.0**119 - 2.0**90, 0x7F7F),
        (2.0**-133, 0x0001),  # smallest subnormal
        (2.0**-134, 0x0000),  # half of it: tie to even (zero)
        (3 * 2.0**-134, 0x0002),  # tie between 1 and 2 quanta: to even
        (2.0**-126, 0x0080),  # smallest normal
        (2.0**-126 - 2.0**-133, 0x007F),  # largest subnormal
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
    ],
)
def test_f64_to_bf16_hand_cases(v, bits):
    assert oracle.f64_to_bf16(v) == bits


def test_f64_to_bf16_nan():
    assert oracle.f64_to_bf16(float("nan")) == 0x7FC0


def test_f64_to_bf16_matches_nearest_search():
    rng = np.random.default_rng(7)
    v = np.concatenate(
        [
            rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
            rng.standard_normal(500) * 2.0**-130,  # subnormal range
            # exact midpoints between neighbouring bf16 values
            (np.arange(1, 2000, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
            * (1 + 2.0**-8),
        ]
    )
    want = nearest_bf16_bits(v)
    got = np.array([oracle.f64_to_bf16(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, want)


def test_e2m1_matches_ocp_table():
    tab = e2m1_table()
    for code in range(16):
        got = oracle.e2m1(code)
        assert got == tab[code], code
        assert math.copysign(1, got) == math.copysign(1, tab[code]), code


def test_e8m0_closed_form():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(128) == 2.0
    assert oracle.e8m0(119) == 2.0**-8
    assert oracle.e8m0(0) == 2.0**-127
    assert oracle.e8m0(254) == 2.0**127
    assert math.isnan(oracle.e8m0(255))


def test_mx_elem_nibble_order_and_scale_block():
    q = np.zeros(32, np.uint8)
    s = np.full(2, 127, np.uint8)
    q[0] = 0x21  # k=0 low nibble 0x1 (0.5), k=1 high nibble 0x2 (1.0)
    q[15] = 0xF7  # k=30: 0x7 (6), k=31: 0xF (-6)
    q[16] = 0x0C  # k=32: 0xC (-2), k=33: 0
    s[1] = 129  # elements 32..63 scaled by 4
    assert oracle.mx_elem(q, s, 0) == 0.5
    assert oracle.mx_elem(q, s, 1) == 1.0
    assert oracle.mx_elem(q, s, 30) == 6.0
    assert oracle.mx_elem(q, s, 31) == -6.0
    assert oracle.mx_elem(q, s, 32) == -8.0
    assert oracle.mx_elem(q, s, 33) == 0.0
    assert oracle.mx_elem(q, s, 2) == 0.0


def test_mx_round_trip_every_code_and_scale():
    """decode then nearest-encode gives the code back, for every non-NaN
    scale byte and every nibble (-0 keeps its sign)."""
    tab = e2m1_table()
    for x in range(0, 255, 7):
        for code in range(16):
            q = np.array([code], np.uint8)
            s = np.array([x], np.uint8)
            v = oracle.mx_elem(q, s, 0)
            scale = 2.0 ** (x - 127)
            cands = [c for c in range(16) if tab[c] * scale == v and math.copysign(1, tab[c]) == math.copysign(1, v)]
            assert cands == [code], (x, code, v)


# IEEE 754 binary32: the largest finite value is (2 - 2^-23) 2^127, so a
# magnitude of 2^128 or more is out of range; 2^-149 is the smallest subnormal.
@pytest.mark.parametrize(
    "code,x,want",
    [
        (0x1, 0, 2.0**-128),  # 0.5 x 2^-127: a subnormal, exact
        (0x9, 0, -(2.0**-128)),
        (0x7, 0, 6 * 2.0**-127),
        (0x3, 1, 1.5 * 2.0**-126),
        (0x7, 252, 6 * 2.0**125),  # 1.5 x 2^127: the largest finite decoded value
        (0x5, 253, 3 * 2.0**126),  # 1.5 x 2^127 again
        (0x6, 253, float("inf")),  # 4 x 2^126 = 2^128: out of range
        (0xE, 253, float("-inf")),
        (0x7, 253, float("inf")),
        (0x3, 254, 1.5 * 2.0**127),
        (0x4, 254, float("inf")),  # 2 x 2^127
        (0xC, 254, float("-inf")),
        (0x0, 254, 0.0),
    ],
)
def test_mx_elem_range_ends(code, x, want):
    """The decoded weight is a value of the MFMA's operand format: every
    e2m1 x 2^(X-127) is exact there except magnitudes >= 2^128, which
    overflow to infinity (scale bytes 253 and 254)."""
    v = oracle.mx_elem(np.array([code], np.uint8), np.array([x], np.uint8), 0)
    assert v == want and math.copysign(1, v) == math.copysign(1, want), (code, x, v)


def test_mx_elem_nan_scale_is_nan_for_every_code():
    """e8m0 0xFF is NaN (OCP MX v1.0): all 32 elements of its block are NaN,
    zeros included."""
    for code in range(16):
        v = oracle.mx_elem(np.array([code], np.uint8), np.array([255], np.uint8), 0)
        assert math.isnan(v), code
