"""Exact-rational helpers for brute-force pins (pure Python, independent of the oracle's C code)."""
from fractions import Fraction

import numpy as np


def e4m3_value(code: int) -> Fraction:
    """Value of an OCP E4M3 byte from its fields (1 sign, 4 exponent bits with bias 7, 3 mantissa bits)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN")
    v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def round_to_f32(x: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) binary32 value of an exact rational."""
    f = np.float32(float(x))  # within one binary32 ulp of x
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        dist = abs(Fraction(float(cand)) - x)
        key = (dist, int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def round_half_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def e5m2_value(code: int) -> Fraction:
    """Value of a finite OCP E5M2 byte from its fields (1 sign, 5 exponent bits with bias 15, 2 mantissa bits)."""
    s, e, m = code >> 7, (code >> 2) & 31, code & 3
    if e == 31:
        raise ValueError("infinity or NaN")
    v = Fraction(m, 1 << 16) if e == 0 else Fraction(4 + m, 4) * Fraction(2) ** (e - 15)
    return -v if s else v
