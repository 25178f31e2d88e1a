"""The oracle's exact sums where binary64 is not enough: means whose correct rounding depends
on bits far below binary64 resolution, the incremental update's binary64 rounding of an exact
sum that sits next to a binary64 tie, and nearest centroids that differ in squared distance
only far below binary64 resolution. Expected values are rational arithmetic on constructed
inputs (tests/_wide_span.py); the first four cases also check that a plain binary64 running
sum gets a share of them wrong, so the inputs do exercise more than binary64. The last one
takes means onto the subnormal grids of binary32 and bfloat16."""
import numpy as np

import oracle
import synth
from tests import _wide_span as ws


def test_centroid_means_beyond_binary64():
    """One cluster of 256 tokens: the centroid is fl32 of the exact mean (paper page, method
    step (1): the centroid update is the mean of the members)."""
    rng = np.random.default_rng(1)
    n, d = 256, 64
    X, exact, rounded = ws.mean_columns(rng, n, d, "f32")
    V = synth.bf16_bits(X.astype(np.float32))
    C = oracle.kmeans_update(V, np.zeros(n, np.int32), np.zeros((1, d), np.float32))
    assert np.array_equal(C[0], np.array(rounded, np.float32))
    naive = np.array([np.float32(ws.running_sum(X[:, c]) / n) for c in range(d)])
    assert np.count_nonzero(naive != C[0]) >= d // 5, np.count_nonzero(naive != C[0])


def test_incremental_sum_rounded_once_to_binary64():
    """decay 0 (no history): C = fl32(fl64(exact sum) / n), one binary64 rounding of the exact
    sum whatever the order of the members."""
    rng = np.random.default_rng(2)
    n, d = 256, 64
    X, expected = ws.f64_tie_columns(rng, n, d)
    V = synth.bf16_bits(X.astype(np.float32))
    lab = np.zeros(n, np.int32)
    C0 = np.full((1, d), 3.0, np.float32)
    _, _, C, M = oracle.kmeans_incremental(V, C0, np.array([7.0], np.float32), 0.0, False, labels=lab)
    assert np.array_equal(C[0], np.array(expected, np.float32))
    assert M[0] == np.float32(n)
    naive = np.array([np.float32(ws.running_sum(X[:, c]) / n) for c in range(d)])
    assert np.count_nonzero(naive != C[0]) >= d // 8, np.count_nonzero(naive != C[0])


def test_block_and_key_means_beyond_binary64():
    """mu = bf16 of each 128-token block's exact mean, kbar = fl32 of the exact key mean over
    the sequence (paper page, method steps (2) and (3))."""
    rng = np.random.default_rng(3)
    N, d = 512, 64
    nb = N // 128
    Vp = np.zeros((N, d))
    mu_exp = np.zeros((nb, d), np.int64)
    for b in range(nb):
        X, _, rounded = ws.mean_columns(rng, 128, d, "bf16")
        Vp[128 * b:128 * (b + 1)] = X
        mu_exp[b] = rounded
    perm = synth.rand_perm(N, 4)
    V = np.zeros_like(Vp)
    V[perm] = Vp                                    # V'[i] = V[perm[i]]
    Kx, _, kbar_exp = ws.mean_columns(rng, N, d, "f32", small=True)
    Q = synth.gen_head("wan", 3, 0, 0, N, d)["Q"]
    q = oracle.quantize(Q, synth.bf16_bits(Kx.astype(np.float32)), synth.bf16_bits(V.astype(np.float32)), perm,
                        oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    assert np.array_equal(q["mu"].astype(np.int64), mu_exp)
    assert np.array_equal(q["kbar"], np.array(kbar_exp, np.float32))
    naive_mu = np.array([[synth.bf16_bits(np.array([ws.running_sum(Vp[128 * b:128 * (b + 1), c]) / 128],
                                                   np.float32))[0] for c in range(d)] for b in range(nb)])
    assert np.count_nonzero(naive_mu != mu_exp) >= nb * d // 5
    naive_k = np.array([np.float32(ws.running_sum(Kx[:, c]) / N) for c in range(d)])
    assert np.count_nonzero(naive_k != q["kbar"]) >= d // 5


def test_nearest_centroid_beyond_binary64():
    """argmin of the exact squared distance, ties to the lowest index (paper page, method step
    (1)), where the candidates' distances agree in every bit binary64 keeps."""
    rng = np.random.default_rng(4)
    N, d, T = 384, 64, 8
    V, C, near = ws.near_tie_tokens(rng, N, d, T)
    lab = oracle.kmeans_assign(V, C)
    Vf = synth.bf16_to_f32(V).astype(np.float64)
    wrong64 = 0
    for t in range(N):
        j = near[t]
        cand = [3 * j, 3 * j + 1, 3 * j + 2]
        ex = [ws.exact_sqdist(Vf[t], C[k]) for k in cand]
        best = cand[int(np.argmin(ex))]                         # first minimum: lowest index
        assert lab[t] == best, (t, lab[t], best)
        f64 = [float(np.sum((Vf[t] - C[k].astype(np.float64)) ** 2)) for k in cand]
        wrong64 += cand[int(np.argmin(f64))] != best
    # every other centroid is far: its binary64 distance exceeds the triple's by more than 32
    D64 = ((Vf[:, None, :] - C[None].astype(np.float64)) ** 2).sum(-1)
    own = D64[np.arange(N)[:, None], 3 * near[:, None] + np.arange(3)[None]].max(1)
    other = np.where((np.arange(3 * T)[None] // 3) == near[:, None], np.inf, D64).min(1)
    assert np.all(other > own + 32)
    assert wrong64 >= N // 4, wrong64


def test_means_on_subnormal_grids():
    """Means of values m 2^-133 (bfloat16 subnormals and the smallest normals): the centroid
    rounds to the binary32 subnormal grid 2^-149 and the block means to the bfloat16 grid
    2^-133, nearest even."""
    from fractions import Fraction as F
    rng = np.random.default_rng(6)
    n, d = 384, 32
    X = ws.tiny_values(rng, n, d).astype(np.float32)
    C = oracle.kmeans_update(synth.bf16_bits(X), np.zeros(n, np.int32), np.zeros((1, d), np.float32))
    exp = np.array([ws.f32_of_tiny(sum(F(float(x)) for x in X[:, c]) / n) for c in range(d)], np.float32)
    assert np.array_equal(C[0], exp)
    assert np.all(np.abs(C[0]) < 2.0 ** -126)
    Q = synth.gen_head("wan", 3, 0, 0, n, d)["Q"]
    q = oracle.quantize(Q, Q, synth.bf16_bits(X), None, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    mexp = np.array([[ws.bf16_of_tiny(sum(F(float(x)) for x in X[128 * b:128 * (b + 1), c]) / 128) for c in range(d)]
                     for b in range(n // 128)])
    assert np.array_equal(q["mu"].astype(np.int64), mexp)
