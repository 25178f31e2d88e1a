"""Pins for the oracle's k-means (paper page, method step (1)): exact argmin with
lowest-index ties, exact rational centroid means, stable argsort, planted-cluster sanity."""
from fractions import Fraction

import numpy as np

import oracle
import synth
from tests._exact import round_to_f32


def _bits_to_fr(h):
    return [Fraction(float(x)) for x in synth.bf16_to_f32(h)]


def test_assign_brute_force_with_ties():
    rng = np.random.default_rng(3)
    N, d, K = 300, 8, 7
    # small integers and halves: many exact ties between clusters
    V = synth.bf16_bits((rng.integers(-4, 5, (N, d)) * 0.5).astype(np.float32))
    C = (rng.integers(-4, 5, (K, d)) * 0.5).astype(np.float32)
    C[3] = C[1]            # duplicate centroid: the lower index must win
    chat = synth.bf16_to_f32(synth.bf16_bits(C))
    got = oracle.kmeans_assign(V, chat)
    Vf = [_bits_to_fr(V[t]) for t in range(N)]
    Cf = [[Fraction(float(x)) for x in chat[k]] for k in range(K)]
    for t in range(N):
        dist = [sum((a - b) ** 2 for a, b in zip(Vf[t], Cf[k])) for k in range(K)]
        want = min(range(K), key=lambda k: (dist[k], k))
        assert got[t] == want, t
    assert not np.any(got == 3)


def test_assign_resolves_near_ties_exactly():
    # two centroids whose binary64 distances agree to ~1e-16 but differ exactly
    d = 128
    rng = np.random.default_rng(9)
    v = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal(d).astype(np.float32) * 100))
    a = v.copy()
    b = v.copy()
    a[0] = (synth.bf16_to_f32(synth.bf16_bits(np.float32(v[0].item() + 2.0 ** -10 * abs(v[0].item())))))
    b[1] = (synth.bf16_to_f32(synth.bf16_bits(np.float32(v[1].item() + 2.0 ** -10 * abs(v[1].item())))))
    da = sum((Fraction(float(x)) - Fraction(float(y))) ** 2 for x, y in zip(v, a))
    db = sum((Fraction(float(x)) - Fraction(float(y))) ** 2 for x, y in zip(v, b))
    sign = (da > db) - (da < db)
    assert oracle.exact_sqdist_cmp(v, a, b) == sign
    lab = oracle.kmeans_assign(synth.bf16_bits(v)[None, :], np.stack([a, b]))
    assert lab[0] == (0 if da <= db else 1)


def test_stable_argsort_matches_numpy():
    rng = np.random.default_rng(4)
    z = rng.integers(0, 37, 5000).astype(np.int32)
    assert np.array_equal(oracle.stable_argsort(z, 37), np.argsort(z, kind="stable"))


def test_update_exact_rational_means():
    rng = np.random.default_rng(6)
    N, d, K = 400, 6, 9
    V = synth.bf16_bits((rng.standard_normal((N, d)) * np.exp2(rng.integers(-20, 20, (N, d)))).astype(np.float32))
    z = rng.integers(0, K - 1, N).astype(np.int32)       # cluster K-1 stays empty
    C0 = rng.standard_normal((K, d)).astype(np.float32)
    C = oracle.kmeans_update(V, z, C0)
    Vf = synth.bf16_to_f32(V)
    for k in range(K):
        idx = np.nonzero(z == k)[0]
        for j in range(d):
            if idx.size == 0:
                assert C[k, j] == C0[k, j]
                continue
            s = sum(Fraction(float(Vf[t, j])) for t in idx)
            assert C[k, j] == round_to_f32(s / idx.size), (k, j)


def test_exact_mean_rounding_bf16_and_f32():
    x = np.array([1.0, 2.0 ** -30, 2.0 ** -30], np.float64)
    # (1 + 2^-29)/3 rounded once
    assert oracle.exact_mean(x, 24) == float(round_to_f32((Fraction(1) + Fraction(2) ** -29) / 3))
    # ties to even at bf16 precision: mean exactly halfway between two bf16 neighbours of 1
    y = np.array([1.0, 1.0 + 2.0 ** -7], np.float64)      # mean = 1 + 2^-8, halfway -> 1.0 (even)
    assert oracle.exact_mean(y, 8) == 1.0
    y2 = np.array([1.0 + 2.0 ** -7, 1.0 + 2.0 ** -6], np.float64)  # mean = 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert oracle.exact_mean(y2, 8) == 1.0 + 2.0 ** -6


def test_planted_clusters_recovered_on_tiny_workload():
    h = synth.gen_head("tiny", 0, 0, 0, 1024, 128)
    V, z_true, centres = h["V"], h["z_true"], h["centres"]
    labels, perm, C = oracle.kmeans(V, 4, 3, cold=False, C=centres)
    inlier = np.ones(V.shape[0], bool)
    inlier[h["outliers"]] = False
    # centres ~5.6 apart with unit noise: the Bayes error is ~0.8 %, so >= 98.5 % of the
    # planted labels and >= 99.5 % agreement with the nearest-true-centre rule
    nearest = oracle.kmeans_assign(V, synth.bf16_to_f32(synth.bf16_bits(centres)))
    assert np.mean(labels[inlier] == z_true[inlier]) >= 0.985
    assert np.mean(labels[inlier] == nearest[inlier]) >= 0.995
    assert np.array_equal(perm, np.argsort(labels, kind="stable"))


def test_cold_start_picks_strided_tokens():
    rng = np.random.default_rng(8)
    N, d, K = 256, 4, 5
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    # one assignment against the cold-start centroids equals assigning to the strided tokens
    labels, perm, C = oracle.kmeans(V, K, 1, cold=True)
    init = synth.bf16_to_f32(V[[(2 * k + 1) * N // (2 * K) for k in range(K)]])
    assert np.array_equal(labels, oracle.kmeans_assign(V, init))


def test_kmeans_cost_brute_force_and_zero():
    """k-means objective (drift statistic): exact rational (1/N) sum ||V_t - bf16(C_z)||^2,
    correctly rounded; zero when every token is its own centroid."""
    from fractions import Fraction
    rng = np.random.default_rng(41)
    N, d, K = 96, 8, 5
    V = synth.bf16_bits((rng.standard_normal((N, d)) * np.exp2(rng.integers(-6, 6, (N, d)))).astype(np.float32))
    C = (rng.standard_normal((K, d)) * 2).astype(np.float32)
    z = rng.integers(0, K, N).astype(np.int32)
    Vf = synth.bf16_to_f32(V)
    Ch = synth.bf16_to_f32(synth.bf16_bits(C))
    tot = Fraction(0)
    for t in range(N):
        for j in range(d):
            df = Fraction(float(Vf[t, j])) - Fraction(float(Ch[z[t], j]))
            tot += df * df
    assert oracle.kmeans_cost(V, C, z) == float(tot / N)
    Vs = synth.bf16_bits(rng.standard_normal((16, d)).astype(np.float32))
    assert oracle.kmeans_cost(Vs, synth.bf16_to_f32(Vs), np.arange(16, dtype=np.int32)) == 0.0


# ---- size-penalised assignment (cheap balancing): distance + fl32(lambda * n_k)
def test_biased_assign_brute_force_with_ties():
    rng = np.random.default_rng(13)
    N, d, K = 300, 8, 7
    V = synth.bf16_bits((rng.integers(-4, 5, (N, d)) * 0.5).astype(np.float32))
    C = (rng.integers(-4, 5, (K, d)) * 0.5).astype(np.float32)
    C[3] = C[1]   # same centroid, same bias: lower index wins
    C[5] = C[2]   # same centroid, smaller bias: the higher index wins
    chat = synth.bf16_to_f32(synth.bf16_bits(C))
    bias = (rng.integers(0, 8, K) * 0.25).astype(np.float32)
    bias[3] = bias[1]
    bias[5] = bias[2] - np.float32(0.25) if bias[2] > 0 else np.float32(0.0)
    bias[2] = bias[5] + np.float32(0.25)
    got = oracle.kmeans_assign_biased(V, chat, bias)
    Vf = [_bits_to_fr(V[t]) for t in range(N)]
    Cf = [[Fraction(float(x)) for x in chat[k]] for k in range(K)]
    Bf = [Fraction(float(b)) for b in bias]
    for t in range(N):
        dist = [sum((a - b) ** 2 for a, b in zip(Vf[t], Cf[k])) + Bf[k] for k in range(K)]
        want = min(range(K), key=lambda k: (dist[k], k))
        assert got[t] == want, t
    assert not np.any(got == 3) and not np.any(got == 2)


def test_balanced_worked_example_on_a_line():
    # centroids 0 and 10 on channel 0; tokens 0..7 and 10. Plain assignment: 0..5 -> 0
    # (5 is a tie, lowest index), 6, 7, 10 -> 1, sizes (6, 3). With lambda = 4 and those
    # sizes the biases are 24 and 12: token t joins cluster 0 iff t^2 + 24 < (10-t)^2 + 12,
    # i.e. t < 4.4, so token 5 moves. New sizes (5, 4), means 2 and 7.
    d = 4
    pos = np.array([0, 1, 2, 3, 4, 5, 6, 7, 10], np.float32)
    Vf = np.zeros((pos.size, d), np.float32)
    Vf[:, 0] = pos
    V = synth.bf16_bits(Vf)
    C = np.zeros((2, d), np.float32)
    C[1, 0] = 10
    lab0, _, _, n0 = oracle.kmeans_balanced(V, 2, 1, False, 0.0, np.zeros(2, np.int32), C)
    assert lab0.tolist() == [0, 0, 0, 0, 0, 0, 1, 1, 1] and n0.tolist() == [6, 3]
    lab, perm, Cn, n = oracle.kmeans_balanced(V, 2, 1, False, 4.0, n0, C)
    assert lab.tolist() == [0, 0, 0, 0, 0, 1, 1, 1, 1]
    assert n.tolist() == [5, 4]
    assert perm.tolist() == list(range(9))
    assert Cn[0, 0] == 2.0 and Cn[1, 0] == 7.0 and not Cn[:, 1:].any()


def test_balanced_lambda_zero_is_plain_kmeans():
    rng = np.random.default_rng(21)
    N, d, K = 1500, 16, 12
    V = synth.bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    lab, perm, C = oracle.kmeans(V, K, 3, cold=True)
    lab2, perm2, C2, n2 = oracle.kmeans_balanced(V, K, 3, True, 0.0, np.full(K, 77, np.int32))
    assert np.array_equal(lab, lab2) and np.array_equal(perm, perm2) and np.array_equal(C, C2)
    assert np.array_equal(n2, np.bincount(lab, minlength=K))


def test_balanced_penalty_evens_out_sizes():
    # a dense blob of 900 tokens beside 4 small ones; from the same start, a moderate size
    # penalty ends with less spread in the cluster sizes than plain iterations do
    rng = np.random.default_rng(5)
    d, K = 8, 8
    centres = rng.standard_normal((5, d)).astype(np.float32) * 6
    sizes = [900, 150, 150, 150, 150]
    Vf = np.concatenate([centres[i] + rng.standard_normal((s, d)).astype(np.float32) for i, s in enumerate(sizes)])
    V = synth.bf16_bits(Vf)
    lab, _, C = oracle.kmeans(V, K, 6, cold=True)
    n0 = np.bincount(lab, minlength=K).astype(np.int32)
    labp, _, _ = oracle.kmeans(V, K, 6, cold=False, C=C)
    plain_spread = np.bincount(labp, minlength=K).std()
    for lam in (0.005, 0.01):
        labb, _, _, nb = oracle.kmeans_balanced(V, K, 6, False, lam, n0, C)
        assert np.array_equal(nb, np.bincount(labb, minlength=K))
        assert nb.std() < plain_spread, lam
