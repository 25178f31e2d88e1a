"""Constructed inputs whose exact sums need more than binary64's 53 significant bits, with
the exact expected results from rational arithmetic (fractions.Fraction):

* columns whose exact mean lies a hair (far below binary64 resolution) above or below a
  binary32 or bfloat16 rounding tie, so that the correctly rounded mean depends on bits a
  binary64 running sum drops;
* columns whose exact sum lies a hair beside a binary64 tie that sits on a binary32 tie
  after the division (the incremental centroid update rounds the sum to binary64 first);
* tokens whose nearest centroids differ in squared distance only below binary64
  resolution.

Every value is an exact bfloat16 value. The columns contain many exactly cancelling pairs of
widely different magnitudes, so a binary64 running sum rounds in many places. Nothing here
implements the method: the expected values are plain rational arithmetic.
"""
from __future__ import annotations

from fractions import Fraction as Fr

import numpy as np

import synth


def _round_even(x: Fr, p: int) -> Fr:
    """x rounded to p significant bits, ties to even (normal range)."""
    if x == 0:
        return Fr(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    g = Fr(2) ** (e - p + 1)
    q = a / g
    n = q.numerator // q.denominator
    r = q - n
    if r > Fr(1, 2) or (r == Fr(1, 2) and n % 2 == 1):
        n += 1
    return (1 if x > 0 else -1) * n * g


def f32_of(x: Fr) -> np.float32:
    return np.float32(float(_round_even(x, 24)))


def bf16_of(x: Fr) -> int:
    return int(synth.bf16_bits(np.array([float(_round_even(x, 8))], np.float32))[0])


def _bf16_value(rng, lo_exp: int, hi_exp: int) -> float:
    """a random bfloat16 value with 8 significant bits, magnitude in [2^lo_exp, 2^(hi_exp+1))"""
    e = int(rng.integers(lo_exp, hi_exp + 1))
    return float(int(rng.integers(128, 256)) * 2.0 ** (e - 7))


def _split_bf16(m: int, shift: int) -> list:
    """m * 2^shift (0 <= m < 2^32) as a sum of at most four bfloat16 values (8-bit chunks)."""
    out = []
    for k in (24, 16, 8, 0):
        c = (m >> k) & 0xFF
        if c:
            out.append(float(c * 2.0 ** (shift + k)))
    return out


def _fill_column(rng, n: int, pieces: list, pair_exp: tuple) -> np.ndarray:
    """n values summing to n + sum(pieces): n // 2 entries 2.0 (and one 1.0 for odd n), the
    given pieces, cancelling pairs +x/-x in the other rows (random magnitudes), zeros where a
    row is left over; rows shuffled."""
    col = np.zeros(n, np.float64)
    rows = rng.permutation(n)
    col[rows[:n // 2]] = 2.0
    k = n // 2
    if n % 2:
        col[rows[k]] = 1.0
        k += 1
    for p in pieces:
        col[rows[k]] = p
        k += 1
    while k + 1 < n:
        x = _bf16_value(rng, *pair_exp) * (1 if rng.random() < 0.5 else -1)
        col[rows[k]], col[rows[k + 1]] = x, -x
        k += 2
    return col


def mean_columns(rng, n: int, ncols: int, target: str, small: bool = False, g: int | None = None):
    """Columns of n values (16 <= n < 2^16) whose exact mean is T + s 2^-g with T a rounding tie
    of the target format ("f32": binary32, "bf16": bfloat16) just above 1, s = +-1 and g well
    below binary64 resolution. Returns (X [n, ncols] float64 of bf16 values, exact means as
    Fractions, correctly rounded means: float32 or bf16 bit patterns). small=True keeps every
    value below 2 in magnitude (n >= 512: pieces below 0.25, pairs below 0.5). g, when given,
    fixes the offset's exponent (else it is drawn from 56..69 for binary32, 55..67 for bf16)."""
    assert 16 <= n < 1 << 16
    X = np.zeros((n, ncols), np.float64)
    exact, rounded = [], []
    for c in range(ncols):
        s = 1 if rng.random() < 0.5 else -1
        if target == "f32":
            odd = 2 * int(rng.integers(0, 1 << (11 if small else 15))) + 1
            tie, fb = 1 + Fr(odd, 1 << 24), 24
            gg = int(rng.integers(56, 70)) if g is None else g
        else:
            odd = 2 * int(rng.integers(0, 64)) + 1
            tie, fb = 1 + Fr(odd, 1 << 8), 8
            gg = int(rng.integers(55, 68)) if g is None else g
        # n T = n + (n odd) 2^-fb and n s 2^-g, each split into bf16 pieces
        pieces = _split_bf16(n * odd, -fb) + [s * v for v in _split_bf16(n, -gg)]
        pair_exp = (-30, -2) if small else (-30, 6)
        X[:, c] = _fill_column(rng, n, pieces, pair_exp)
        m = tie + s * Fr(1, 1 << gg)
        assert sum(Fr(float(v)) for v in X[:, c]) == n * m
        exact.append(m)
        rounded.append(f32_of(m) if target == "f32" else bf16_of(m))
    return X, exact, rounded


def f64_tie_columns(rng, n: int, ncols: int):
    """Columns of n values whose exact sum is X + h + s t: X = n T with T a binary32 tie, h
    half a binary64 unit of X and t far smaller, so fl64(exact sum) is X + 2h for s = +1 and X
    for s = -1, and fl32(fl64(sum) / n) is T's upper neighbour for s = +1 and T's even
    neighbour for s = -1. Returns (X [n, ncols] float64 of bf16 values, expected binary32
    results of fl32(fl64(S) / n))."""
    p = n.bit_length() - 1
    assert n == 1 << p and n >= 128
    out = np.zeros((n, ncols), np.float64)
    exp = []
    for c in range(ncols):
        s = 1 if rng.random() < 0.5 else -1
        odd = 2 * int(rng.integers(0, 1 << 15)) + 1
        T = 1 + Fr(odd, 1 << 24)
        h = Fr(2) ** (p - 53)
        t = Fr(2) ** (p - 53 - int(rng.integers(10, 25)))
        pieces = _split_bf16(odd, p - 24) + [float(h), float(s * t)]
        out[:, c] = _fill_column(rng, n, pieces, (-30, 6))
        S = n * T + h + s * t
        assert sum(Fr(float(v)) for v in out[:, c]) == S
        S64 = _round_even(S, 53)
        exp.append(f32_of(S64 / n))
    return out, exp


def running_sum(col: np.ndarray) -> float:
    """binary64 running sum in row order (what a plain accumulator computes)."""
    s = 0.0
    for v in col:
        s += float(v)
    return s


def near_tie_tokens(rng, N: int, d: int, ntriples: int, tiny_exp: int = -20):
    """Tokens and centroids whose squared distances tie in every bit binary64 keeps.

    Centroid triple j (indices 3j, 3j+1, 3j+2) shares a base vector b_j (bf16 values of
    magnitude about 1 on the base channels) and adds L = 2^10 on a "far" channel; the token
    near triple j is b_j plus tiny values (2^t or 2^(t+1), t = tiny_exp) on a few "tiny"
    channels where the centroids hold 0 or a tiny offset (2^(t-1) or 2^t); the exponent span
    of tokens and centroids together is 10 - (t - 1). Every distance from such a token to its triple is L^2
    plus a sum of squares of order 2^-40: equal after binary64 rounding, different exactly.
    Triples alternate between a three-way near tie (all three within 2^-36) and a two-way one
    (the third centroid 64 further away). Returns (V bf16 bits [N, d], C0 float32
    [3 ntriples, d], which triple each token is near)."""
    far = [0, 1, 2]
    tiny = list(range(3, 11))
    base = list(range(11, d))
    L = 2.0 ** 10
    C = np.zeros((3 * ntriples, d), np.float64)
    bvec = np.zeros((ntriples, d), np.float64)
    for j in range(ntriples):
        bvec[j, base] = [_bf16_value(rng, -1, 0) * (1 if rng.random() < 0.5 else -1) for _ in base]
        for m in range(3):
            C[3 * j + m] = bvec[j]
        C[3 * j + 0, far[0]] = L
        C[3 * j + 1, far[0]] = -L
        C[3 * j + 2, far[1]] = L
        # tiny offsets on a few tiny channels: each centroid its own pattern
        for m in range(3):
            for ch in rng.choice(tiny, 3, replace=False):
                C[3 * j + m, ch] = float(rng.choice([2.0 ** (tiny_exp - 1), -(2.0 ** (tiny_exp - 1)), 2.0 ** tiny_exp]))
        if j % 2 == 1:
            C[3 * j + 2, far[2]] = 8.0  # the third one clearly further: a two-way near tie
    near = rng.integers(0, ntriples, N)
    V = bvec[near].copy()
    for t in range(N):
        for ch in rng.choice(tiny, 4, replace=False):
            V[t, ch] = float(rng.choice([2.0 ** tiny_exp, -(2.0 ** tiny_exp), 2.0 ** (tiny_exp + 1)]))
    return synth.bf16_bits(V.astype(np.float32)), C.astype(np.float32), near


def exact_sqdist(v: np.ndarray, c: np.ndarray) -> Fr:
    return sum((Fr(float(a)) - Fr(float(b))) ** 2 for a, b in zip(v, c))


def tiny_values(rng, n: int, d: int) -> np.ndarray:
    """n x d bfloat16 values m 2^-133 (m in 1..255, random signs): bfloat16 subnormals and the
    smallest normals, whose means round on the subnormal grids of binary32 and bfloat16."""
    m = rng.integers(1, 256, (n, d)).astype(np.float64)
    return m * 2.0 ** -133 * np.where(rng.random((n, d)) < 0.6, 1.0, -1.0)


def f32_of_tiny(x: Fr) -> np.float32:
    """binary32 nearest to x, ties to even, on the subnormal grid 2^-149 below 2^-126."""
    if abs(x) >= Fr(2) ** -126:
        return f32_of(x)
    return np.float32(float(Fr(round(x * Fr(2) ** 149)) / Fr(2) ** 149))


def bf16_of_tiny(x: Fr) -> int:
    """bfloat16 nearest to x, ties to even, on the subnormal grid 2^-133 below 2^-126."""
    if abs(x) >= Fr(2) ** -126:
        return bf16_of(x)
    v = Fr(round(x * Fr(2) ** 133)) / Fr(2) ** 133
    return int(synth.bf16_bits(np.array([float(v)], np.float32))[0]) | (0x8000 if x < 0 and v == 0 else 0)
