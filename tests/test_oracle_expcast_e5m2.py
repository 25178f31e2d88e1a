"""Pins for ExpCast with E5M2 probability bytes (the paper page's future directions: carry
ExpCast to other floating-point formats such as E5M2, each with its own affine
coefficients and error bound).

Derivation (the E4M3 argument of the paper page's ExpCast step, redone for E5M2): a
positive normal E5M2 byte read as an integer is 4 log2 v + 60 + eps2(m) with
eps2(m) = m - 4 log2(1 + m/4). Scaling probabilities by 2^15 puts p = 1 at code
4*15 + 60 = 120, so the direct byte of u = log2 p <= 0 is clip(Round(4u + 120 + beta2),
0, 120), i.e. the single FMA fma(acc, 4 sigma, fl32(fl32(120 + beta2) - 4 m')). beta2 is
the minimax centre of eps2 (-0.172; -0.17 used). The per-row total-variation bound has
the E4M3 form with the octave split into 4 codes: W2 = (1 + max|eps2|)/4 and
TV <= tanh(W2 ln2 / 4) = 5.80 %, plus the underflow tail (codes < 4, u < -30).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests._exact import e5m2_value, e4m3_value, round_half_even, round_to_f32

BETA2 = np.float32(oracle.BETA_E5M2)
C02 = np.float32(np.float32(120.0) + BETA2)


def _eps2(m):
    return m - 4 * np.log2(1 + np.asarray(m, np.float64) / 4)


def test_e5m2_codec_against_format_definition():
    got = oracle.e5m2_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        e, m = (c >> 2) & 31, c & 3
        if e == 31:
            if m == 0:
                assert np.isinf(got[c]) and (got[c] < 0) == bool(c >> 7)
            else:
                assert np.isnan(got[c])
            continue
        assert got[c] == float(e5m2_value(c)), c
    pos = got[:124]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 57344.0 and pos[1] == 2.0 ** -16


def test_e5m2_byte_is_affine_in_log2():
    for c in range(4, 124):  # positive normal codes
        v = float(e5m2_value(c))
        assert c == pytest.approx(4 * math.log2(v) + 60 + float(_eps2(c & 3)), abs=1e-12), c
    # equality exactly at m = 0 (powers of two)
    for e in range(1, 31):
        assert 4 * e == 4 * math.log2(float(e5m2_value(4 * e))) + 60


def test_beta2_is_the_minimax_centre_of_eps2():
    m = np.linspace(0.0, 4.0, 400001)
    eps = _eps2(m)
    centre = (eps.max() + eps.min()) / 2
    eps_int = _eps2(np.arange(4))
    centre_int = (eps_int.max() + eps_int.min()) / 2
    assert centre == pytest.approx(-0.1720, abs=2e-4)
    assert centre_int == pytest.approx(-0.1699, abs=2e-4)
    assert abs(centre - float(BETA2)) < 0.005 and abs(centre_int - float(BETA2)) < 0.005


def _closed_form_fractions2(beta: float):
    """Measure over f in [0, 1) of rne(4 f + beta) - rne(4 (2^f - 1)) in {0, +1, -1}: inside a
    normal octave u = k + f the exact code is 4(k + 30) + rne(4(2^f - 1)) and the direct code
    4(k + 30) + rne(4 f + beta)."""
    pts = {0.0, 1.0}
    for j in range(-1, 6):
        x = math.log2(1 + (j + 0.5) / 4)
        if 0 < x < 1:
            pts.add(x)
        y = (j + 0.5 - beta) / 4
        if 0 < y < 1:
            pts.add(y)
    pts = sorted(pts)
    acc = {}
    for a, b in zip(pts[:-1], pts[1:]):
        f = (a + b) / 2
        diff = round(4 * f + beta) - round(4 * (2 ** f - 1))
        acc[diff] = acc.get(diff, 0.0) + (b - a)
    return acc


def _nearest_e5m2_code(v: np.ndarray) -> np.ndarray:
    """Exp-then-cast with an exact exponential: nearest positive E5M2 code (ties to even mantissa)."""
    grid = oracle.e5m2_decode(np.arange(124, dtype=np.uint8))
    idx = np.clip(np.searchsorted(grid, v, side="left"), 1, 123)
    lo, hi = grid[idx - 1], grid[idx]
    pick_hi = ((hi - v) < (v - lo)) | (((hi - v) == (v - lo)) & (idx % 2 == 0))
    out = np.where(pick_hi, idx, idx - 1)
    return np.where(v <= grid[0], 0, out)


def test_oracle_agreement_per_octave_matches_closed_form():
    fr = _closed_form_fractions2(float(BETA2))
    assert set(k for k, v in fr.items() if v > 0) <= {-1, 0, 1}
    assert sum(fr.values()) == pytest.approx(1.0)
    n = 1 << 15
    for k in range(-29, 0):
        u = (k + (np.arange(n, dtype=np.float64) + 0.5) / n).astype(np.float32)
        direct = oracle.expcast(u, np.float32(4.0), C02).astype(np.int64)
        exact = _nearest_e5m2_code(np.exp2(u.astype(np.float64) + 15.0)).astype(np.int64)
        d = direct - exact
        assert np.all(np.abs(d) <= 1), k
        assert np.mean(d == 0) == pytest.approx(fr[0], abs=5e-4), k
    print("[e5m2] direct code == exact-then-cast code on %.2f %% of each octave (+1: %.2f %%, -1: %.2f %%)"
          % (100 * fr[0], 100 * fr.get(1, 0.0), 100 * fr.get(-1, 0.0)))


def test_expcast_e5m2_landmarks():
    ex = lambda u: int(np.asarray(oracle.expcast(np.float32(u), np.float32(4.0), C02)).reshape(-1)[0])
    assert ex(0.0) == 120                                 # p = 1 -> 2^15
    assert float(e5m2_value(120)) == 2.0 ** 15
    assert ex(-15.0) == 60 and float(e5m2_value(60)) == 1.0   # p = 2^-15 -> 1.0
    assert ex(-29.0) == 4 and ex(-31.0) == 0              # last normal octave, then underflow
    assert ex(2.0) == 120                                 # clamp above


def _tv_rows(rng, rows, keys, sigma, spread):
    acc = (rng.standard_normal((rows, keys)) * spread).astype(np.float32)
    sig = np.float32(sigma)
    mp = (sig * acc.max(axis=1)).astype(np.float32)
    bias = (C02 - np.float32(4.0) * mp).astype(np.float32)
    codes = oracle.expcast(acc, np.float32(4.0) * sig, bias[:, None])
    q = oracle.e5m2_decode(codes)
    logits = sig.astype(np.float64) * acc.astype(np.float64)
    p = np.exp2(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    qn = q / q.sum(axis=1, keepdims=True)
    tv = 0.5 * np.abs(qn - p).sum(axis=1)
    under = codes < 4
    tau = (p * under).sum(axis=1) + (qn * under).sum(axis=1)
    return tv, tau, under.any(axis=1)


def test_tv_bound_e5m2_closed_form():
    eps_int = [float(_eps2(k)) for k in range(4)]
    W2 = (1 + max(abs(e) for e in eps_int)) / 4
    assert W2 == pytest.approx(0.33497, abs=1e-5)
    assert math.tanh(W2 * math.log(2) / 4) == pytest.approx(0.05801, abs=5e-5)


@pytest.mark.parametrize("spread", [0.5, 3.0, 12.0])
def test_oracle_rows_obey_tv_bound_e5m2(spread):
    eps_int = [float(_eps2(k)) for k in range(4)]
    bound = math.tanh((1 + max(abs(e) for e in eps_int)) / 4 * math.log(2) / 4)
    tv, tau, has_under = _tv_rows(np.random.default_rng(12), 3000, 256, 0.37, spread)
    assert np.all(tv <= bound + tau + 1e-6)
    clean = ~has_under
    assert clean.any()
    assert np.all(tv[clean] <= bound + 1e-6)
    assert 0.003 < np.median(tv) < bound


def test_online_e5m2_codes_and_output_match_exact_recomputation():
    """Brute force on a tiny head: every E5M2 byte of the online loop from exact rationals,
    and the emulated output from those bytes by a direct (non-online) formula."""
    rng = np.random.default_rng(22)
    N, d = 256, 16
    Q = synth.bf16_bits((rng.standard_normal((N, d)) * 4).astype(np.float32))
    K = synth.bf16_bits((rng.standard_normal((N, d)) * 4 + 1).astype(np.float32))
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    perm = rng.permutation(N).astype(np.int32)
    q = oracle.quantize(Q, K, V, perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    rows = np.array([3, 130, 255], np.int32)
    nb = N // 128
    dec4 = {c: e4m3_value(c) for c in range(256) if (c & 0x7F) != 0x7F}
    codes_all = np.zeros((rows.size, N), np.int64)
    m_all = np.zeros((rows.size, nb))
    for blk in range(nb):
        _, codes, mm = oracle.attention_emul(q, rows, beta=float(BETA2), mode=oracle.MODE_EXPCAST_E5M2,
                                             dump_block=blk, want_m=True)
        for ri, i in enumerate(rows):
            I = i // 128
            m = None
            for j in range(blk + 1):
                sigma = np.float32(q["sQ"][I] * q["sK"][j])
                accs = [round_to_f32(sum(dec4[int(q["Qq"][i, c])] * dec4[int(q["Kq"][j * 128 + t, c])]
                                         for c in range(d))) for t in range(128)]
                mnew = np.float32(sigma * max(accs))
                m = mnew if m is None else max(m, mnew)
            assert mm[ri, blk] == m
            bias = np.float32(C02 - np.float32(4.0) * m)
            s4 = np.float32(np.float32(4.0) * sigma)
            for t in range(128):
                tt = round_to_f32(Fraction(float(accs[t])) * Fraction(float(s4)) + Fraction(float(bias)))
                want = min(max(round_half_even(Fraction(float(tt))), 0), 120)
                assert codes[ri, t] == want, (blk, i, t)
            codes_all[ri, blk * 128:(blk + 1) * 128] = codes[ri]
            m_all[ri, blk] = mm[ri, blk]
    # output from the bytes: O = sV * sum_j 2^(m_j - m_last) sum_t dec(c) (dec(Rq) + mu~_j) / l
    O = oracle.attention_emul(q, rows, beta=float(BETA2), mode=oracle.MODE_EXPCAST_E5M2)
    R = oracle.e4m3_decode(q["Vq"]) + np.repeat(q["mu_scaled"].astype(np.float64), 128, axis=0)
    for ri in range(rows.size):
        w = oracle.e5m2_decode(codes_all[ri].astype(np.uint8)) * np.repeat(np.exp2(m_all[ri] - m_all[ri, -1]), 128)
        want = q["sV"].astype(np.float64) * (w @ R) / w.sum()
        assert np.allclose(O[ri], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
