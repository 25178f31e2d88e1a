"""Pins for the oracle's E4M3 codec.

The paper page's prerequisite on E4M3 fixes the format (1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits) and states that the byte read as an integer equals
8*log2(v) + 56 + eps(m): an affine function of the stored value's logarithm.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import e4m3_value


def test_decode_landmarks():
    # values that a wrong bias or a swapped field would move
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert dec[0x38] == 1.0           # exponent field 7 = bias -> 1.0
    assert dec[0x7E] == 448.0         # largest finite value
    assert dec[0x08] == 2.0 ** -6     # smallest normal
    assert dec[0x01] == 2.0 ** -9     # smallest subnormal
    assert dec[0x78] == 256.0         # code 120 = 2^8 (the ExpCast ceiling)
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert dec[0x80] == 0.0 and math.copysign(1.0, dec[0x80]) < 0


def test_decode_all_codes_against_fields():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert Fraction(dec[c]) == e4m3_value(c), hex(c)


def test_positive_grid_is_monotone_with_eight_steps_per_binade():
    dec = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(dec) > 0)
    for e in range(1, 16):
        vals = dec[8 * e: 8 * e + 8] if e < 15 else dec[120:127]
        steps = np.diff(vals)
        assert np.all(steps == steps[0])  # uniform spacing inside a binade


def test_byte_is_log_affine_on_normal_codes():
    """byte = 8 log2 v + 56 + eps(m), eps(m) = m - 8 log2(1 + m/8) in [-0.68, 0], eps(0) = 0."""
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    n = 0
    for c in range(8, 127):
        m = c & 7
        eps = m - 8 * math.log2(1 + m / 8)
        assert abs(c - (8 * math.log2(dec[c]) + 56 + eps)) < 1e-12, c
        n += 1
    assert n == 119
    eps_int = [m - 8 * math.log2(1 + m / 8) for m in range(8)]
    assert eps_int[0] == 0.0 and min(eps_int) == pytest.approx(-0.67970, abs=1e-5)


def test_encode_roundtrip_and_ties():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    enc = oracle.e4m3_encode(np.array([dec[c] for c in codes], np.float32))
    assert list(enc) == codes
    # exact midpoints between neighbours go to the even code
    for c in range(0, 126):
        mid = np.float32((dec[c] + dec[c + 1]) / 2)
        assert float(mid) == (dec[c] + dec[c + 1]) / 2  # representable in binary32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == want, c
        assert oracle.e4m3_encode(np.array([-mid]))[0] == want | 0x80, c


def test_encode_brute_force_random_and_saturation():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(4000) * np.exp2(rng.integers(-12, 10, 4000))).astype(np.float32)
    x = np.concatenate([x, np.float32([448.0, 449.0, 463.9, 464.0, 1e6, -500.0, 1e-6, -1e-6, 0.0, -0.0])])
    enc = oracle.e4m3_encode(x)
    pos = [e4m3_value(c) for c in range(127)]
    for xi, ci in zip(x, enc):
        a = abs(Fraction(float(xi)))
        if a >= 448:
            want = 126
        else:
            best = min(range(127), key=lambda c: (abs(pos[c] - a), c % 2))
            want = best
        if math.copysign(1.0, float(xi)) < 0:
            want |= 0x80
        assert ci == want, (xi, hex(ci), hex(want))
