"""Pins for the oracle's quantiser and attention emulation.

* Quantiser on exactly representable inputs reproduces every planted code, scale,
  block mean and channel mean (paper page, method step (2); study notes 2-2).
* With the probability quantiser switched off, the emulated pipeline equals exact
  attention for any joint K/V permutation, with and without block-mean removal: the
  permutation is exact (study notes 2-1, P'V' = PV) and the mean is restored exactly
  from the row sums (study notes 2-3, P_ij V'_j = P_ij R_j + r_ij mu_j^T).
* The probability bytes inside the online loop equal a from-scratch exact-rational
  recomputation (brute force) on a tiny head.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests._construct import representable_head
from tests._exact import e4m3_value, round_half_even, round_to_f32


@pytest.mark.parametrize("permute", [False, True])
@pytest.mark.parametrize("vsmooth", [False, True])
def test_quantizer_exact_construction(permute, vsmooth):
    h = representable_head(N=512, d=32, seed=1 + 2 * permute + vsmooth, permute=permute, vsmooth=vsmooth)
    flags = oracle.FLAG_KSMOOTH | (oracle.FLAG_VSMOOTH if vsmooth else 0)
    q = oracle.quantize(h["Q"], h["K"], h["V"], h["perm"], flags)
    e = h["exp"]
    cL = oracle.log2e_over_sqrt_d(32)
    assert np.array_equal(q["Qq"], e["Qq"])
    assert np.array_equal(q["sQ"], (e["sQ_raw"] * cL).astype(np.float32))
    assert np.array_equal(q["Kq"], e["Kq"])
    assert np.array_equal(q["sK"], e["sK"])
    assert np.array_equal(q["kbar"], e["kbar"])
    assert np.array_equal(q["Vq"], e["Vq"])
    assert np.array_equal(q["sV"], e["sV"])
    if vsmooth:
        assert np.array_equal(synth.bf16_to_f32(q["mu"]), e["mu"])
        assert np.array_equal(q["mu_scaled"], (e["mu"] * 32).astype(np.float32))


def test_log2e_constant():
    # fl32(log2(e)/sqrt(d)) against binary64 evaluation (differs only if a tie were near)
    for d in (64, 128, 32):
        c = oracle.log2e_over_sqrt_d(d)
        assert abs(float(c) - np.log2(np.e) / np.sqrt(d)) <= np.spacing(c) / 2


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("permute", [False, True])
@pytest.mark.parametrize("vsmooth", [False, True])
def test_identity_probabilities_equal_exact_attention(permute, vsmooth):
    h = representable_head(N=512, d=32, seed=10 + 2 * permute + vsmooth, permute=permute, vsmooth=vsmooth)
    flags = oracle.FLAG_KSMOOTH | (oracle.FLAG_VSMOOTH if vsmooth else 0)
    q = oracle.quantize(h["Q"], h["K"], h["V"], h["perm"], flags)
    rows = np.arange(0, 512, 7, dtype=np.int32)
    O = oracle.attention_emul(q, rows, mode=oracle.MODE_EXACT_PROB)
    Oex = oracle.attention_exact(h["Q"], h["K"], h["V"], rows)
    assert _rel_l2(O, Oex) < 2e-5
    if vsmooth:
        # dropping the restored mean term is a large error: the pin sees the r*mu term
        Onr = oracle.attention_emul(q, rows, mode=oracle.MODE_EXACT_PROB, restore_mean=False)
        assert _rel_l2(Onr, Oex) > 1e-2


def test_exact_attention_permutation_invariance_and_direct_form():
    rng = np.random.default_rng(2)
    N, d = 384, 16
    Q = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32) * 2)
    K = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32) * 2)
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    rows = np.arange(0, N, 5, dtype=np.int32)
    O = oracle.attention_exact(Q, K, V, rows)
    p = rng.permutation(N)
    Op = oracle.attention_exact(Q, K[p], V[p], rows)
    assert np.max(np.abs(O - Op)) < 1e-12
    q, k, v = (synth.bf16_to_f32(x).astype(np.float64) for x in (Q, K, V))
    s = q[rows] @ k.T / np.sqrt(d)
    w = np.exp(s - s.max(1, keepdims=True))
    direct = (w / w.sum(1, keepdims=True)) @ v
    assert np.max(np.abs(O - direct)) < 1e-12


def test_online_codes_match_exact_rational_recomputation():
    rng = np.random.default_rng(21)
    N, d = 384, 16
    Q = synth.bf16_bits((rng.standard_normal((N, d)) * 3).astype(np.float32))
    K = synth.bf16_bits((rng.standard_normal((N, d)) * 3 + 1).astype(np.float32))
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    perm = rng.permutation(N).astype(np.int32)
    q = oracle.quantize(Q, K, V, perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    rows = np.array([0, 77, 200, 383], np.int32)
    beta = np.float32(-0.35)
    C0 = np.float32(np.float32(120.0) + beta)
    nb = N // 128
    dec = {c: e4m3_value(c) for c in range(256) if (c & 0x7F) != 0x7F}
    for blk in range(nb):
        _, codes, mm = oracle.attention_emul(q, rows, beta=float(beta), mode=oracle.MODE_EXPCAST,
                                             dump_block=blk, want_m=True)
        for ri, i in enumerate(rows):
            I = i // 128
            m = None
            for j in range(blk + 1):
                sigma = np.float32(q["sQ"][I] * q["sK"][j])
                accs = []
                for t in range(128):
                    s = sum(dec[int(q["Qq"][i, c])] * dec[int(q["Kq"][j * 128 + t, c])] for c in range(d))
                    accs.append(round_to_f32(s))
                mx = max(accs)
                mnew = np.float32(sigma * mx)
                m = mnew if m is None else max(m, mnew)
                assert mm[ri, j] == m
            bias = np.float32(C0 - np.float32(8.0) * m)
            s8 = np.float32(np.float32(8.0) * sigma)
            for t in range(128):
                tt = round_to_f32(Fraction(float(accs[t])) * Fraction(float(s8)) + Fraction(float(bias)))
                want = min(max(round_half_even(Fraction(float(tt))), 0), 120)
                assert codes[ri, t] == want, (blk, i, t)


def test_vsmooth_beats_plain_on_tiny_workload():
    """Pages' claim (news page, V-Smooth section): sorting + block-mean removal lowers the value error."""
    h = synth.gen_head("tiny", 0, 0, 0, 1024, 128)
    labels, perm, _ = oracle.kmeans(h["V"], 8, 4, cold=True)
    rows = np.arange(0, 1024, 3, dtype=np.int32)
    Oex = oracle.attention_exact(h["Q"], h["K"], h["V"], rows)
    O_plain, _ = oracle.pipeline(h["Q"], h["K"], h["V"], rows, vsmooth=False, expcast_on=False)
    O_vs, _ = oracle.pipeline(h["Q"], h["K"], h["V"], rows, vsmooth=True, expcast_on=False, perm=perm)
    O_vc, _ = oracle.pipeline(h["Q"], h["K"], h["V"], rows, vsmooth=True, expcast_on=True, perm=perm)
    e_plain, e_vs, e_vc = _rel_l2(O_plain, Oex), _rel_l2(O_vs, Oex), _rel_l2(O_vc, Oex)
    assert e_vs < e_plain
    assert e_vc < 0.1


def _pow2_f32(u: np.float32) -> np.float32:
    """fl32(2^u) for a binary32 u, from a 60-digit decimal evaluation (correctly rounded unless
    2^u lies within 1e-50 relative of a binary32 midpoint)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    v = (Decimal(float(u)) * Decimal(2).ln()).exp()
    return round_to_f32(Fraction(v))


def _e4m3_nearest_even(x: Fraction) -> int:
    """RNE of a nonnegative rational to an E4M3 code (saturating), by brute force over the table."""
    best = None
    for c in range(0x7F):
        v = e4m3_value(c)
        key = (abs(v - x), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_exp_then_cast_codes_rowsums_and_output_match_exact_recomputation():
    """Exp-then-cast probabilities (the plain-FP8 and V-Smooth-only paths): for every key,
    p = fl32(2^u) with u = fl32(fl32(sigma acc) - m'), byte = e4m3(256 p), and the row sum is
    256 sum p while the values are weighted by the decoded bytes (study notes 2-3: the row
    sum the kernel already keeps). Recomputed from scratch with decimals and rationals: every
    byte equals the oracle's, and the output agrees to 1e-12 relative. An e-based
    exponential, a different probability scale or a row sum taken from the bytes fails."""
    rng = np.random.default_rng(33)
    N, d = 256, 16
    Q = synth.bf16_bits((rng.standard_normal((N, d)) * 2).astype(np.float32))
    K = synth.bf16_bits((rng.standard_normal((N, d)) * 2).astype(np.float32))
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    q = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH)
    rows = np.array([3, 130, 255], np.int32)
    nb = N // 128
    dec = {c: e4m3_value(c) for c in range(256) if (c & 0x7F) != 0x7F}
    O_or = oracle.attention_emul(q, rows, mode=oracle.MODE_EXP_THEN_CAST, restore_mean=False)
    dumps = [oracle.attention_emul(q, rows, mode=oracle.MODE_EXP_THEN_CAST, restore_mean=False, dump_block=j)[1]
             for j in range(nb)]
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    for ri, i in enumerate(rows):
        I = i // 128
        m, A, l = None, [Fraction(0)] * d, Fraction(0)
        for j in range(nb):
            sigma = np.float32(q["sQ"][I] * q["sK"][j])
            accs = [round_to_f32(sum(dec[int(q["Qq"][i, c])] * dec[int(q["Kq"][j * 128 + t, c])] for c in range(d)))
                    for t in range(128)]
            mnew = np.float32(sigma * max(accs))
            mp = mnew if m is None else max(m, mnew)
            alpha = Fraction(0) if m is None else Fraction((Decimal(float(m) - float(mp)) * Decimal(2).ln()).exp())
            r, pv = Fraction(0), [Fraction(0)] * d
            for t in range(128):
                u = np.float32(np.float32(sigma * accs[t]) - mp)
                P = _pow2_f32(u)
                code = _e4m3_nearest_even(Fraction(float(np.float32(256.0) * P)))
                assert dumps[j][ri, t] == code, (i, j, t)
                r += 256 * Fraction(float(P))
                for c in range(d):
                    pv[c] += dec[code] * dec[int(q["Vq"][j * 128 + t, c])]
            l = alpha * l + r
            A = [alpha * a + x for a, x in zip(A, pv)]
            m = mp
        want = [float(Fraction(float(q["sV"][c])) * A[c] / l) for c in range(d)]
        assert np.allclose(O_or[ri], want, rtol=1e-12, atol=1e-14 * max(abs(x) for x in want)), (i, O_or[ri], want)
