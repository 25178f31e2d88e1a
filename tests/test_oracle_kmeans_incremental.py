"""Pins of the oracle's cross-step incremental centroid update (oracle.kmeans_incremental; the
paper page's weakness list: update centroids incrementally across denoising steps instead of
clustering each step from scratch).

* a worked example on small integers, derived by hand (decayed masses, one empty cluster);
* decay 0 with the labels kept equals the plain centroid update (exact member means), and with
  re-assignment equals one warm Lloyd iteration -- labels, permutation and centroids;
* decay 1 pools the steps: two steps' members give their pooled mean, up to the one binary32
  rounding the first step's centroid carries.
"""
from fractions import Fraction

import numpy as np

import oracle
import synth


def _bf(x):
    return synth.bf16_bits(np.asarray(x, np.float32))


def test_worked_example():
    # cluster 0: mass 4 at (0, 0), members (1, 0), (2, 2); cluster 1: mass 2 at (10, 4), members
    # (9, 4), (12, 4), (15, 7); cluster 2: mass 3 at (7, 7), no members. decay 1/2:
    #   A = (2, 1, 1.5); den = A + n = (4, 4, -); num_0 = 2*(0,0) + (3,2) = (3,2) -> C_0 = (0.75, 0.5)
    #   num_1 = 1*(10,4) + (36,15) = (46,19) -> C_1 = (11.5, 4.75); C_2 kept, M_2 = 1.5
    V = _bf([[1, 0], [2, 2], [9, 4], [12, 4], [15, 7]])
    C = np.array([[0, 0], [10, 4], [7, 7]], np.float32)
    M = np.array([4, 2, 3], np.float32)
    lab, perm, Cn, Mn = oracle.kmeans_incremental(V, C, M, 0.5, False, labels=[0, 0, 1, 1, 1])
    assert np.array_equal(Cn, np.array([[0.75, 0.5], [11.5, 4.75], [7, 7]], np.float32))
    assert np.array_equal(Mn, np.array([4, 4, 1.5], np.float32))
    assert np.array_equal(lab, [0, 0, 1, 1, 1]) and np.array_equal(perm, [0, 1, 2, 3, 4])


def test_decay_zero_is_the_plain_update_and_one_lloyd_iteration():
    w = synth.gen("wan", seed=31, B=1, H=1, N=2048, d=64)
    V = w["V"][0, 0]
    rng = np.random.default_rng(3)
    K = 37
    C0 = (rng.standard_normal((K, 64)) * 2).astype(np.float32)
    M0 = rng.uniform(0, 50, K).astype(np.float32)
    lab0 = rng.integers(0, K - 2, 2048).astype(np.int32)          # two clusters stay empty
    lab, perm, C, M = oracle.kmeans_incremental(V, C0, M0, 0.0, False, labels=lab0)
    want = oracle.kmeans_update(V, lab0, C0)
    assert np.array_equal(C, want)
    assert np.array_equal(M, np.bincount(lab0, minlength=K).astype(np.float32))
    assert np.array_equal(perm, np.argsort(lab0, kind="stable"))
    lab, perm, C, M = oracle.kmeans_incremental(V, C0, M0, 0.0, True)
    l1, p1, c1 = oracle.kmeans(V, K, 1, cold=False, C=C0)
    assert np.array_equal(lab, l1) and np.array_equal(perm, p1) and np.array_equal(C, c1)


def test_decay_one_pools_two_steps():
    rng = np.random.default_rng(5)
    N, d, K = 1024, 32, 8
    V1 = _bf(rng.standard_normal((N, d)) * 3)
    V2 = _bf(rng.standard_normal((N, d)) * 3 + 1)
    lab = rng.integers(0, K, N).astype(np.int32)
    C0 = np.zeros((K, d), np.float32)
    _, _, C1, M1 = oracle.kmeans_incremental(V1, C0, np.zeros(K, np.float32), 1.0, False, labels=lab)
    _, _, C2, M2 = oracle.kmeans_incremental(V2, C1, M1, 1.0, False, labels=lab)
    n = np.bincount(lab, minlength=K)
    assert np.array_equal(M2, (2 * n).astype(np.float32))
    f1, f2 = synth.bf16_to_f32(V1).astype(np.float64), synth.bf16_to_f32(V2).astype(np.float64)
    for k in range(K):
        pooled = (f1[lab == k].sum(0) + f2[lab == k].sum(0)) / (2 * n[k])
        # the carried centroid C1 = fl32(mean_1) is off by at most half an ulp, weighted n/2n
        tol = np.spacing(np.abs(C1[k]).astype(np.float32)) / 4 + np.spacing(np.abs(C2[k]).astype(np.float32)) / 2
        assert np.all(np.abs(C2[k] - pooled) <= tol * (1 + 1e-9)), k


def test_quotient_rounding_on_exact_rationals():
    """decay 1/4 on a head of random values: every new centroid is the binary32 nearest to
    (A C + S) / (A + n) with A C + S and A + n taken in binary64, recomputed with fractions."""
    rng = np.random.default_rng(8)
    N, d, K = 512, 16, 5
    V = _bf(rng.standard_normal((N, d)) * 5)
    C0 = (rng.standard_normal((K, d)) * 5).astype(np.float32)
    M0 = rng.uniform(1, 100, K).astype(np.float32)
    lab = rng.integers(0, K, N).astype(np.int32)
    _, _, C, M = oracle.kmeans_incremental(V, C0, M0, 0.25, False, labels=lab)
    f = synth.bf16_to_f32(V).astype(np.float64)
    from tests._exact import round_to_f32
    for k in range(K):
        A = 0.25 * float(M0[k])
        n = int((lab == k).sum())
        den = A + n
        assert M[k] == np.float32(den)
        for j in range(d):
            S = float(sum(Fraction(float(x)) for x in f[lab == k, j]))   # exact, then binary64
            num = A * float(C0[k, j]) + S
            assert C[k, j] == round_to_f32(Fraction(num) / Fraction(den)), (k, j)
