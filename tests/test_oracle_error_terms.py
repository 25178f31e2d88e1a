"""The oracle's split of the quantised output's error into a probability term and a value
term, O_q - O = (W - P) V + W (V_q - V) (the paper page's error analysis of low-bit
attention: the probability error and the value error add up to the output error).

Pins: the two terms sum to the emulated output's error; the effective weights of an
ExpCast path sum to one per row (its row sum is the sum of its decoded probabilities);
the exact probabilities reproduce the oracle's binary64 attention; with exactly
representable inputs and unquantised probabilities both terms vanish.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._construct import representable_head


def _rel(a, ref):
    return float(np.linalg.norm(a) / np.linalg.norm(ref))


@pytest.mark.parametrize("vsmooth", [False, True])
def test_error_terms_vanish_with_identity_quantisers(vsmooth):
    h = representable_head(N=512, d=32, seed=30 + vsmooth, permute=True, vsmooth=vsmooth)
    flags = oracle.FLAG_KSMOOTH | (oracle.FLAG_VSMOOTH if vsmooth else 0)
    q = oracle.quantize(h["Q"], h["K"], h["V"], h["perm"], flags)
    rows = np.arange(0, 512, 5, dtype=np.int32)
    T1, T2, E, O = oracle.error_terms(h["Q"], h["K"], h["V"], q, h["perm"], rows, mode=oracle.MODE_EXACT_PROB)
    assert _rel(T1, O) < 2e-5
    assert _rel(T2, O) < 1e-12
    assert np.abs(T1 + T2 - E).max() <= 1e-12 * np.abs(O).max()


@pytest.mark.parametrize("mode,vsmooth", [(oracle.MODE_EXPCAST, True), (oracle.MODE_EXPCAST, False),
                                          (oracle.MODE_EXP_THEN_CAST, False)])
def test_error_terms_sum_to_output_error(mode, vsmooth):
    w = synth.gen("tiny")
    Q, K, V = (w[k][0, 0] for k in ("Q", "K", "V"))
    _, perm, _ = oracle.kmeans(V, 8, 4, cold=True)
    perm = perm if vsmooth else None
    flags = oracle.FLAG_KSMOOTH | (oracle.FLAG_VSMOOTH if vsmooth else 0)
    q = oracle.quantize(Q, K, V, perm, flags)
    rows = np.arange(0, 1024, 3, dtype=np.int32)
    T1, T2, E, O = oracle.error_terms(Q, K, V, q, perm, rows, mode=mode)
    assert np.abs(T1 + T2 - E).max() <= 1e-11 * np.abs(O).max()
    assert np.abs(O - oracle.attention_exact(Q, K, V, rows)).max() <= 1e-12 * np.abs(O).max()
    _, W = oracle.attention_emul(q, rows, mode=mode, want_weights=True)
    if mode == oracle.MODE_EXPCAST:
        assert np.abs(W.sum(axis=1) - 1.0).max() < 1e-12
    else:  # the row sum uses the binary32 probabilities, the values their E4M3 codes
        assert np.abs(W.sum(axis=1) - 1.0).max() < 0.05
    assert W.min() >= 0.0


def test_exp_then_cast_with_mean_restoration_is_rejected():
    w = synth.gen("tiny")
    Q, K, V = (w[k][0, 0] for k in ("Q", "K", "V"))
    q = oracle.quantize(Q, K, V, None, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    with pytest.raises(ValueError):
        oracle.error_terms(Q, K, V, q, None, np.arange(4, dtype=np.int32), mode=oracle.MODE_EXP_THEN_CAST)


def test_error_terms_wan_head():
    """Report on head 0 of the Wan-shaped workload (64 sampled rows): V-Smooth must shrink
    the value term of the ExpCast path; the figures are printed."""
    w = synth.gen("wan", heads=[0])
    Q, K, V, Vp = (w[k][0, 0] for k in ("Q", "K", "V", "V_prev"))
    _, _, Cw = oracle.kmeans(Vp, 550, 1, cold=True)
    _, perm, _ = oracle.kmeans(V, 550, 2, cold=False, C=Cw)
    rows = np.sort(np.random.default_rng(5).choice(V.shape[0], 64, replace=False)).astype(np.int32)
    res = {}
    for name, vs, mode in (("vc", True, oracle.MODE_EXPCAST), ("expcast", False, oracle.MODE_EXPCAST),
                           ("plain", False, oracle.MODE_EXP_THEN_CAST)):
        p = perm if vs else None
        q = oracle.quantize(Q, K, V, p, oracle.FLAG_KSMOOTH | (oracle.FLAG_VSMOOTH if vs else 0))
        T1, T2, E, O = oracle.error_terms(Q, K, V, q, p, rows, mode=mode)
        res[name] = (_rel(T1, O), _rel(T2, O), _rel(E, O))
        assert np.abs(T1 + T2 - E).max() <= 1e-11 * np.abs(O).max()
    print("[error terms] relative norms (probability, value, total): " +
          "; ".join("%s %.4f%% %.4f%% %.4f%%" % (k, 100 * a, 100 * b, 100 * c) for k, (a, b, c) in res.items()))
    assert res["vc"][1] < res["expcast"][1]
