"""Pins for the preprocessing the pages' fused quantiser absorbs: RoPE and the Q/K
Hadamard rotation (paper page, core method: the fused kernel takes in RoPE, the mean,
the gather, the Hadamard rotation and the quantiser; the news page's FP8 background:
a Hadamard rotation spreads channel outliers).

RoPE reading: interleaved pairs (2i, 2i+1), caller's binary32 cos/sin tables, binary32
products and sum/difference, result rounded to bf16. Hadamard reading: unnormalised
Sylvester matrix by the fast transform (ascending stages), 1/d folded into sQ'.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth
from tests._exact import round_to_f32


def _bf16_of_fraction(x: Fraction) -> int:
    """bf16 bits of an exactly known binary32 value (round to nearest even on 16 bits)."""
    f = np.float32(float(x))
    assert Fraction(float(f)) == x
    return int(synth.bf16_bits(np.array([f], np.float32))[0])


def _tables(rng, N, d):
    ang = rng.uniform(-np.pi, np.pi, (N, d // 2))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _position_tables(N, d, base=10000.0):
    """1-D rotary tables: angle t * base^(-2i/d) for token t and pair i."""
    ang = np.arange(N)[:, None] * base ** (-2.0 * np.arange(d // 2)[None, :] / d)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_rope_identity_and_quarter_turn():
    rng = np.random.default_rng(1)
    N, d = 64, 16
    x = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    one, zero = np.ones((N, d // 2), np.float32), np.zeros((N, d // 2), np.float32)
    assert np.array_equal(oracle.rope(x, one, zero), x)
    y = oracle.rope(x, zero, one)                       # (a, b) -> (-b, a)
    xf = synth.bf16_to_f32(x)
    assert np.array_equal(synth.bf16_to_f32(y)[:, 0::2], -xf[:, 1::2])
    assert np.array_equal(synth.bf16_to_f32(y)[:, 1::2], xf[:, 0::2])


def test_rope_matches_exact_rational_recomputation():
    rng = np.random.default_rng(2)
    N, d = 24, 8
    x = synth.bf16_bits((rng.standard_normal((N, d)) * 3).astype(np.float32))
    c, s = _tables(rng, N, d)
    got = oracle.rope(x, c, s)
    xf = synth.bf16_to_f32(x)
    for t in range(N):
        for i in range(d // 2):
            a, b = Fraction(float(xf[t, 2 * i])), Fraction(float(xf[t, 2 * i + 1]))
            cc, ss = Fraction(float(c[t, i])), Fraction(float(s[t, i]))
            ac, bs, as_, bc = (Fraction(float(round_to_f32(v))) for v in (a * cc, b * ss, a * ss, b * cc))
            want0 = _bf16_of_fraction(Fraction(float(round_to_f32(ac - bs))))
            want1 = _bf16_of_fraction(Fraction(float(round_to_f32(as_ + bc))))
            assert got[t, 2 * i] == want0 and got[t, 2 * i + 1] == want1, (t, i)


def test_rope_is_a_rotation():
    rng = np.random.default_rng(3)
    N, d = 256, 64
    x = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    c, s = _tables(rng, N, d)
    y = synth.bf16_to_f32(oracle.rope(x, c, s)).astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    z = (xf[:, 0::2] + 1j * xf[:, 1::2]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    assert np.allclose(y[:, 0::2], z.real, rtol=0, atol=2 ** -7 * np.abs(xf).max())
    assert np.allclose(y[:, 1::2], z.imag, rtol=0, atol=2 ** -7 * np.abs(xf).max())
    # pair norms preserved up to bf16 rounding
    n_in = np.hypot(xf[:, 0::2], xf[:, 1::2])
    n_out = np.hypot(y[:, 0::2], y[:, 1::2])
    assert np.all(np.abs(n_out - n_in) <= 2 ** -7 * n_in + 1e-30)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_fwht_equals_sylvester_matrix_on_integers(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, (40, d)).astype(np.float32)      # every partial sum exact
    H = scipy.linalg.hadamard(d).astype(np.float64)
    y = oracle.fwht_rows(x)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ H.T)
    assert np.array_equal(oracle.fwht_rows(y).astype(np.float64), d * x.astype(np.float64))   # H H = d I


def test_fwht_rounding_bound_on_random_rows():
    rng = np.random.default_rng(7)
    d = 128
    x = (rng.standard_normal((200, d)) * np.exp2(rng.integers(-8, 8, (200, d)))).astype(np.float32)
    y = oracle.fwht_rows(x).astype(np.float64)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(d).astype(np.float64).T
    bound = 7 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y - ref) <= bound)


def test_quantize_with_rope_equals_rope_then_quantize():
    rng = np.random.default_rng(4)
    N, d = 384, 64
    w = synth.gen("wan", seed=9, B=1, H=1, N=N, d=d)
    Q, K, V = (w[k][0, 0] for k in ("Q", "K", "V"))
    c, s = _tables(rng, N, d)
    perm = rng.permutation(N).astype(np.int32)
    flags = oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH | oracle.FLAG_HADAMARD
    a = oracle.quantize(Q, K, V, perm, flags, rope_cos=c, rope_sin=s)
    b = oracle.quantize(oracle.rope(Q, c, s), oracle.rope(K, c, s), V, perm, flags)
    for k in ("Qq", "sQ", "Kq", "sK", "Vq", "sV", "mu", "mu_scaled", "kbar"):
        assert np.array_equal(a[k], b[k]), k


def test_hadamard_quantiser_codes_from_rotated_rows():
    """Q codes of the Hadamard path are the plain path's quantiser applied to the rotated
    rows; sQ' carries the extra exact factor 1/d."""
    w = synth.gen("tiny")
    Q, K, V = (w[k][0, 0] for k in ("Q", "K", "V"))
    d = Q.shape[1]
    h = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH | oracle.FLAG_HADAMARD)
    p = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH)
    rot = oracle.fwht_rows(synth.bf16_to_f32(Q))
    blk = rot[:128]
    a = np.abs(blk).max()
    assert h["sQ"][0] == np.float32(np.float32(np.float32(a / np.float32(448.0)) * oracle.log2e_over_sqrt_d(d)) / d)
    assert np.array_equal(h["Qq"][:128], oracle.e4m3_encode(blk * np.float32(np.float32(448.0) / a)))
    assert np.array_equal(h["kbar"], p["kbar"]) and np.array_equal(h["Vq"], p["Vq"])


def test_rope_hadamard_pipeline_matches_exact_attention():
    """Unquantised probabilities: the emulated output equals binary64 attention on the
    RoPE'd inputs up to the FP8 Q/K quantisation, with and without the rotation (a wrong
    1/d folding would show as a softmax temperature off by a factor d)."""
    w = synth.gen("tiny")
    Q, K, V = (w[k][0, 0] for k in ("Q", "K", "V"))
    N, d = Q.shape
    c, s = _position_tables(N, d)
    rows = np.arange(0, N, 9, dtype=np.int32)
    Oex = oracle.attention_exact(oracle.rope(Q, c, s), oracle.rope(K, c, s), V, rows)
    err = {}
    for had in (False, True):
        q = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH | (oracle.FLAG_HADAMARD if had else 0),
                            rope_cos=c, rope_sin=s)
        O = oracle.attention_emul(q, rows, mode=oracle.MODE_EXACT_PROB, restore_mean=False)
        err[had] = np.linalg.norm(O - Oex) / np.linalg.norm(Oex)
    print("[rope] score-path error without / with rotation: %.4f / %.4f" % (err[False], err[True]))
    assert err[False] < 0.1 and err[True] < 0.1
    assert 0.5 < err[True] / err[False] < 2.0


def test_hadamard_tames_channel_outliers():
    """With a few outlier channels in Q and K the rotation lowers the score error of the
    FP8 path (the reason the pages' fused chain carries it)."""
    rng = np.random.default_rng(6)
    N, d = 512, 128
    Qf = rng.standard_normal((N, d)).astype(np.float32)
    Kf = rng.standard_normal((N, d)).astype(np.float32)
    ch = rng.choice(d, 4, replace=False)
    Qf[:, ch] *= 40.0
    Kf[:, ch] *= 40.0
    Q, K = synth.bf16_bits(Qf), synth.bf16_bits(Kf)
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    rows = np.arange(0, N, 4, dtype=np.int32)
    Oex = oracle.attention_exact(Q, K, V, rows)
    errs = {}
    for had in (False, True):
        q = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH | (oracle.FLAG_HADAMARD if had else 0))
        O = oracle.attention_emul(q, rows, mode=oracle.MODE_EXACT_PROB, restore_mean=False)
        errs[had] = np.linalg.norm(O - Oex) / np.linalg.norm(Oex)
    print("[hadamard] score-path error without / with rotation: %.4f / %.4f" % (errs[False], errs[True]))
    assert errs[True] < errs[False]
