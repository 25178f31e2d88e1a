"""Pin of the oracle's output rounding (binary64 -> bfloat16, nearest, ties to even, one
rounding): the output format of the attention epilogue (O = bf16(s_V A / l)). Checked against
a brute-force nearest-value search on exact rationals, on exact ties, on values just off a tie,
on the double-rounding trap (a value that a detour through binary32 would move onto a tie),
on subnormals and on signed zeros."""
from fractions import Fraction

import numpy as np

import oracle


def _bf16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))


def _nearest_bf16_bits(x: float) -> int:
    """Brute force: among the finite bf16 values around x, the nearest; ties to the even
    significand; the sign of zero follows x."""
    fx = Fraction(x)
    f32 = np.float32(x)  # only to find the neighbourhood
    b = int(np.array([f32], np.float32).view(np.uint32)[0] >> 16)
    cands = []
    for c in range(b - 3, b + 4):
        c &= 0xFFFF
        if (c & 0x7F80) == 0x7F80:  # inf / NaN
            continue
        cands.append(c)
    best = None
    for c in cands:
        dist = abs(_bf16_value(c) - fx)
        key = (dist, c & 1)  # equal distance: the even significand wins
        if best is None or key < best[0]:
            best = (key, c)
    bits = best[1]
    if _bf16_value(bits) == 0:
        bits = 0x8000 if np.signbit(x) else 0x0000
    return bits


def _cases():
    rng = np.random.default_rng(3)
    xs = []
    # random doubles over the normal and subnormal bf16 range
    xs += list(rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000)))
    # exact ties between neighbours, and values just off them
    for _ in range(500):
        e = int(rng.integers(-133, 120))
        m = int(rng.integers(0, 256))
        a = float(_bf16_value((max(0, min(0x7F7F, ((e + 127) << 7) | (m & 0x7F))))))
        nxt = np.nextafter(np.float32(a), np.float32(np.inf))
        b = float(_bf16_value(int(np.array([np.float32(a)], np.float32).view(np.uint32)[0] >> 16) + 1))
        mid = (a + b) / 2  # exact in binary64
        xs += [mid, -mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
        # double-rounding trap: just above the tie by less than half a binary32 ulp there, so a
        # detour through binary32 lands on the tie and then rounds to even instead of up
        ulp32 = float(nxt) - a if nxt != np.float32(a) else 0.0
        if ulp32 > 0:
            xs.append(mid + ulp32 / 4)
            xs.append(-(mid + ulp32 / 4))
    xs += [0.0, -0.0, 1e-300, -1e-300, 2.0 ** -134, 2.0 ** -133, 1.5 * 2.0 ** -133]
    return [float(x) for x in xs if np.isfinite(x) and abs(x) < 3.3e38]


def test_bf16_round_is_the_nearest_even_value():
    xs = _cases()
    got = oracle.bf16_round(np.array(xs, np.float64))
    want = np.array([_nearest_bf16_bits(x) for x in xs], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], hex(int(got[i])), hex(int(want[i]))) for i in bad[:5]]


def test_double_rounding_through_binary32_is_not_what_the_oracle_does():
    # the trap value rounds up directly, but to even (down) through binary32
    a = 1.0 + 2.0 ** -7           # bf16 value with an odd significand
    b = 1.0 + 2.0 ** -6
    x = (a + b) / 2 + 2.0 ** -28  # above the tie by less than half a binary32 ulp (2^-24)
    assert np.float32(x) == np.float32((a + b) / 2)
    assert int(oracle.bf16_round(np.array([x]))[0]) == _nearest_bf16_bits(x)
    assert _bf16_value(_nearest_bf16_bits(x)) == Fraction(b)
