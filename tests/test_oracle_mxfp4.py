"""Pins for the 4-bit residual path (paper page, method step (2): the residual quantised to
4 bits on workstation parts; the pages' 4-bit results show V-Smooth helping most there).

Reading: OCP MXFP4 -- E2M1 elements, one power-of-two (E8M0) scale per group of 32 keys of
a channel, scale = the smallest 2^e with amax <= 6 * 2^e, ties to even mantissa; groups =
within each 64-key half of a 128-key block, keys 16g..16g+15 and 32+16g..32+16g+15.
"""
import numpy as np
import pytest

import oracle
import synth


def _e2m1_field(c):
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    v = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
    return -v if s else v


def _group(t):
    return 2 * (t >> 6) + ((t >> 4) & 1)


def test_e2m1_codec():
    got = oracle.e2m1_decode(np.arange(16))
    assert list(got) == [_e2m1_field(c) for c in range(16)]
    grid = [_e2m1_field(c) for c in range(8)]
    # ties go to the even mantissa
    for x, want in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6), (6.0, 7),
                    (-0.1, 0), (-0.3, 9), (-6.0, 15)]:
        assert oracle.e2m1_encode(x)[()] == want, x
    rng = np.random.default_rng(1)
    for x in rng.uniform(-6, 6, 2000):
        c = int(oracle.e2m1_encode(x)[()])
        best = min(abs(abs(x) - g) for g in grid)
        assert abs(abs(_e2m1_field(c)) - abs(x)) == best


def _mx_head(rng, N, d):
    """V' whose every group is exactly representable: E2M1 codes times 2^e, with one element of
    magnitude 4 or 6 per group so that e is the scale the rule must find."""
    nb = N // 128
    e = rng.integers(-6, 6, (nb, d, 4))
    codes = rng.integers(0, 16, (N, d)).astype(np.uint8)
    codes[(codes & 7) == 0] = 0                      # no negative zero
    for b in range(nb):
        for g in range(4):
            ts = [t for t in range(128) if _group(t) == g]
            for c in range(d):
                codes[b * 128 + rng.choice(ts), c] = rng.choice([6, 7, 14, 15])
    vals = np.array([_e2m1_field(int(c)) for c in codes.ravel()]).reshape(N, d)
    grp = np.array([_group(t) for t in range(128)])
    scale = np.exp2(e[:, :, grp].transpose(0, 2, 1).reshape(N, d).astype(np.float64))
    return vals * scale, codes, (e + 127).astype(np.uint8)


def test_mx_quantiser_exact_construction():
    rng = np.random.default_rng(2)
    N, d = 256, 16
    Vv, codes, sc = _mx_head(rng, N, d)
    V = synth.bf16_bits(Vv.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(V), Vv.astype(np.float32))
    Q = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    K = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    q = oracle.quantize(Q, K, V, None, oracle.FLAG_MXFP4)
    assert np.array_equal(q["Vq"], codes)
    assert np.array_equal(q["Vs"], sc)
    assert np.all(q["sV"] == 1.0)
    # zero groups: scale 2^0 and zero codes
    q0 = oracle.quantize(Q, K, np.zeros_like(V), None, oracle.FLAG_MXFP4)
    assert np.all(q0["Vs"] == 127) and np.all(q0["Vq"] == 0)


def test_mx_scale_is_smallest_unclipped_power_of_two():
    rng = np.random.default_rng(3)
    N, d = 128, 8
    V = synth.bf16_bits((rng.standard_normal((N, d)) * np.exp2(rng.integers(-4, 4, (1, d)))).astype(np.float32))
    q = oracle.quantize(V, V, V, None, oracle.FLAG_MXFP4)
    Vf = synth.bf16_to_f32(V).astype(np.float64)
    grp = np.array([_group(t) for t in range(128)])
    for c in range(d):
        for g in range(4):
            a = np.abs(Vf[grp == g, c]).max()
            e = int(q["Vs"][0, c, g]) - 127
            assert a <= 6 * 2.0 ** e and a > 6 * 2.0 ** (e - 1)
            rec = oracle.e2m1_decode(q["Vq"][grp == g, c]) * 2.0 ** e
            assert np.all(np.abs(rec - Vf[grp == g, c]) <= 2.0 ** e)   # half of the largest E2M1 step


def test_mx_value_term_vanishes_for_representable_values():
    """Unquantised probabilities, V exactly representable in MXFP4: the value term of the
    error split is zero and the terms still sum to the emulated error (pins the emulator's
    MXFP4 decode and group scales)."""
    rng = np.random.default_rng(4)
    N, d = 256, 16
    Vv, _, _ = _mx_head(rng, N, d)
    V = synth.bf16_bits(Vv.astype(np.float32))
    Q = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    K = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    q = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH | oracle.FLAG_MXFP4)
    rows = np.arange(0, N, 5, dtype=np.int32)
    T1, T2, E, O = oracle.error_terms(Q, K, V, q, None, rows, mode=oracle.MODE_EXACT_PROB)
    assert np.abs(T2).max() == 0.0
    assert np.abs(T1 + T2 - E).max() <= 1e-12 * np.abs(O).max()


def test_mx_vsmooth_helps_the_4bit_value_error():
    """Pages: V-Smooth gains most on the 4-bit path. Value term of the error split on a
    Wan-shaped head (64 rows): MXFP4 with block-mean removal below MXFP4 without, and both
    above the 8-bit value term."""
    w = synth.gen("wan", heads=[0], N=8192)
    Q, K, V, Vp = (w[k][0, 0] for k in ("Q", "K", "V", "V_prev"))
    _, _, Cw = oracle.kmeans(Vp, 64, 1, cold=True)
    _, perm, _ = oracle.kmeans(V, 64, 2, cold=False, C=Cw)
    rows = np.sort(np.random.default_rng(5).choice(V.shape[0], 64, replace=False)).astype(np.int32)
    val = {}
    for name, flags, p in (("mx_vs", oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH | oracle.FLAG_MXFP4, perm),
                           ("mx", oracle.FLAG_KSMOOTH | oracle.FLAG_MXFP4, None),
                           ("e4m3_vs", oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH, perm)):
        q = oracle.quantize(Q, K, V, p, flags)
        T1, T2, E, O = oracle.error_terms(Q, K, V, q, p, rows, mode=oracle.MODE_EXPCAST)
        val[name] = np.linalg.norm(T2) / np.linalg.norm(O)
        assert np.abs(T1 + T2 - E).max() <= 1e-11 * np.abs(O).max()
    print("[mxfp4] value term: MXFP4 %.4f%%, MXFP4 + V-Smooth %.4f%%, E4M3 + V-Smooth %.4f%%"
          % (100 * val["mx"], 100 * val["mx_vs"], 100 * val["e4m3_vs"]))
    assert val["mx_vs"] < val["mx"]
    assert val["e4m3_vs"] < val["mx_vs"]
