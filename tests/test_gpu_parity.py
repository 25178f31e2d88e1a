"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: ExpCast function bytes, quantiser outputs (codes, scales, means), k-means
labels / permutation / centroids. Floating point: attention output within relative L2
2e-3 of the oracle's emulation. In-kernel probability bytes: every disagreement must
be a single code and lie inside the band that the matrix cores' score accumulation
can move (gfx950 FP8 MFMA sums products in groups of 8 K-slots, each product
truncated 13 bits below the group's largest exponent sum; the oracle's scores are the
exactly rounded dot products).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402

vc = pytest.importorskip("bit_attention_video_online_amd")
from tests.gpu_util import bf16_bits, gpu_quantize, mu_pack_expected, mx_unpack, rel_l2, to_dev, to_dev_bf16, vq_rowmajor  # noqa: E402

BETA = oracle.BETA_E4M3
BETA2 = oracle.BETA_E5M2
# Output tolerance. The VC path (E4M3 bytes): relative L2 2e-3 against the emulation. The
# matrix core's score rounding moves a few bytes across a code boundary (see the in-kernel
# byte test); with E5M2 bytes one code step is a factor 2^(1/4) instead of 2^(1/8), so the
# same moved byte changes its probability (2^(1/4) - 1) / (2^(1/8) - 1) = 2.09 times as much.
TOL = 2e-3
TOL_E5M2 = TOL * (2 ** 0.25 - 1) / (2 ** 0.125 - 1)
FLAGS_ALL = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH


def _ok():
    return torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not _ok():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ ExpCast function
def test_expcast_function_bitexact():
    rng = np.random.default_rng(7)
    n = 1 << 20
    acc = (rng.standard_normal(n) * np.exp2(rng.integers(-6, 14, n))).astype(np.float32)
    s8 = (8.0 * np.exp2(rng.uniform(-16, -2, n))).astype(np.float32)
    mprime = (rng.uniform(-50, 50, n)).astype(np.float32)
    bias = (np.float32(np.float32(120.0) + np.float32(BETA)) - np.float32(8.0) * mprime).astype(np.float32)
    # exact ties and clamp edges
    k = rng.integers(-3, 124, 4096).astype(np.float32)
    acc = np.concatenate([acc, k + np.float32(0.5), k, np.float32([120.5, 121.5, -0.5, -0.51, 0.49, 119.65, 1e9, -1e9])])
    s8 = np.concatenate([s8, np.ones(2 * 4096 + 8, np.float32)])
    bias = np.concatenate([bias, np.zeros(2 * 4096 + 8, np.float32)])
    want = oracle.expcast(acc, s8, bias)
    out = torch.empty(acc.size, dtype=torch.uint8, device="cuda")
    vc.vc_debug_expcast(to_dev(acc), to_dev(s8), to_dev(bias), out)
    got = out.cpu().numpy()
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]


def test_mfma_peak_kernel_counts_every_instruction():
    # fixed operands: E4M3 1.0 (A) and 0.5 (B); per round each lane's 16 outputs of the four
    # chains gain 64 * (0.5 + 0.5 + 1 + 0.25), so the lane sum is exactly 2304 per round
    grid, iters = 300, 37
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    vc.vc_debug_mfma_peak(grid, iters, False, out)
    assert torch.all(out == 2304.0 * iters)
    vc.vc_debug_mfma_peak(grid, iters, True, out)
    assert torch.isfinite(out).all()


# ------------------------------------------------------------------ quantiser
def _compare_quant(out, q_or, b, h, vsmooth):
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    assert np.array_equal(g["Qq"][b, h], q_or["Qq"])
    assert np.array_equal(g["sQ"][b, h], q_or["sQ"])
    assert np.array_equal(g["Kq"][b, h], q_or["Kq"])
    assert np.array_equal(g["sK"][b, h], q_or["sK"])
    assert np.array_equal(vq_rowmajor(g["Vq"])[b, h], q_or["Vq"])
    assert np.array_equal(g["sV"][b, h], q_or["sV"])
    assert np.array_equal(g["mu_scaled"][b, h], q_or["mu_scaled"])
    if vsmooth:
        assert np.array_equal(bf16_bits(out["mu"])[b, h], q_or["mu"])
    assert np.array_equal(g["mu_pack"][b, h], mu_pack_expected(q_or["mu_scaled"]))


@pytest.mark.parametrize("flags", [FLAGS_ALL, vc.VC_F_KSMOOTH, vc.VC_F_VSMOOTH, 0])
@pytest.mark.parametrize("use_perm", [True, False])
def test_quantize_bitexact_tiny(flags, use_perm):
    w = synth.gen("tiny")
    N = w["meta"]["N"]
    perm = synth.rand_perm(N, 0)[None, None] if use_perm else None
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm, flags)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], None if perm is None else perm[0, 0], flags)
    _compare_quant(out, q_or, 0, 0, bool(flags & 2))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [128, 384])
def test_quantize_bitexact_shapes(d, N):
    """Single block and ragged (3-block) heads, two batches x three heads, both head sizes."""
    B, H = 2, 3
    w = synth.gen("wan", seed=5, B=B, H=H, N=N, d=d)
    perm = np.stack([np.stack([synth.rand_perm(N, 9, b, h) for h in range(H)]) for b in range(B)])
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm, FLAGS_ALL)
    for b in range(B):
        for h in range(H):
            q_or = oracle.quantize(w["Q"][b, h], w["K"][b, h], w["V"][b, h], perm[b, h], FLAGS_ALL)
            _compare_quant(out, q_or, b, h, True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rope,had", [(True, False), (False, True), (True, True)])
def test_quantize_rope_hadamard_bitexact(d, rope, had):
    """RoPE (video-grid angle tables) and the Q/K Hadamard rotation inside the quantiser,
    ragged 3-block heads, permuted keys: every output bit-exact against the oracle."""
    B, H, N = 1, 2, 384
    w = synth.gen("wan", seed=8, B=B, H=H, N=N, d=d)
    perm = np.stack([np.stack([synth.rand_perm(N, 11, b, h) for h in range(H)]) for b in range(B)])
    tabs = synth.rope_tables(N, d, (3, 8, 16)) if rope else None
    flags = FLAGS_ALL | (vc.VC_F_HADAMARD if had else 0)
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm, flags, rope=tabs)
    for h in range(H):
        q_or = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], perm[0, h],
                               oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH | (oracle.FLAG_HADAMARD if had else 0),
                               rope_cos=None if tabs is None else tabs[0], rope_sin=None if tabs is None else tabs[1])
        _compare_quant(out, q_or, 0, h, True)


@pytest.mark.parametrize("e5m2", [False, True])
def test_attention_after_rope_hadamard_matches_emulation(e5m2):
    w = synth.gen("tiny")
    N, d = 1024, 128
    perm = synth.rand_perm(N, 2)
    tabs = synth.rope_tables(N, d, (4, 16, 16))
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm[None, None], FLAGS_ALL | vc.VC_F_HADAMARD, rope=tabs)
    O, _ = _gpu_attention(out, N, d, 1, 1, True, True, e5m2=e5m2)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], perm,
                           oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH | oracle.FLAG_HADAMARD,
                           rope_cos=tabs[0], rope_sin=tabs[1])
    rows = np.arange(N, dtype=np.int32)
    O_or = oracle.attention_emul(q_or, rows, beta=BETA2 if e5m2 else BETA,
                                 mode=oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST)
    err = rel_l2(_o_f64(O[0, 0]), O_or)
    print("[rope+hadamard %s] rel-L2 vs emulation %.3e" % ("e5m2" if e5m2 else "e4m3", err))
    assert err <= (TOL_E5M2 if e5m2 else TOL), err


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("vsmooth", [False, True])
def test_quantize_mxfp4_bitexact(d, vsmooth):
    """4-bit (MXFP4) value residual: codes, group scales and the rest of the quantiser
    outputs bit-exact against the oracle; ragged 3-block heads with permuted keys."""
    B, H, N = 1, 2, 384
    w = synth.gen("wan", seed=14, B=B, H=H, N=N, d=d)
    perm = np.stack([np.stack([synth.rand_perm(N, 15, b, h) for h in range(H)]) for b in range(B)])
    flags = vc.VC_F_KSMOOTH | (vc.VC_F_VSMOOTH if vsmooth else 0) | vc.VC_F_MXFP4
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm, flags)
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    codes, scales = mx_unpack(g["Vq"])
    for h in range(H):
        q_or = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], perm[0, h], int(flags))
        assert np.array_equal(codes[0, h], q_or["Vq"]), h
        assert np.array_equal(scales[0, h], q_or["Vs"]), h
        for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu_scaled"):
            assert np.array_equal(g[k][0, h], q_or[k]), (h, k)
        assert np.array_equal(g["mu_pack"][0, h], mu_pack_expected(q_or["mu_scaled"]))


def test_quantize_exact_construction():
    from tests._construct import representable_head
    hd = representable_head(N=512, d=128, seed=3)
    out = gpu_quantize(hd["Q"][None, None], hd["K"][None, None], hd["V"][None, None], hd["perm"][None, None], FLAGS_ALL)
    e = hd["exp"]
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    assert np.array_equal(g["Qq"][0, 0], e["Qq"])
    assert np.array_equal(g["Kq"][0, 0], e["Kq"])
    assert np.array_equal(vq_rowmajor(g["Vq"])[0, 0], e["Vq"])
    assert np.array_equal(g["sV"][0, 0], e["sV"])
    assert np.array_equal(g["sK"][0, 0], e["sK"])


# ------------------------------------------------------------------ k-means
def _gpu_cluster(V, K, iters, cold, C0=None):
    B, H, N, d = V.shape
    C = torch.zeros((B, H, K, d), dtype=torch.float32, device="cuda") if C0 is None else to_dev(C0.astype(np.float32))
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    vc.vc_cluster(to_dev_bf16(V), K, iters, cold, C, lab, perm)
    torch.cuda.synchronize()
    return lab.cpu().numpy(), perm.cpu().numpy(), C.cpu().numpy()


def test_cluster_bitexact_tiny_cold():
    w = synth.gen("tiny")
    lab, perm, C = _gpu_cluster(w["V"], 8, 4, True)
    l_or, p_or, c_or = oracle.kmeans(w["V"][0, 0], 8, 4, cold=True)
    assert np.array_equal(lab[0, 0], l_or)
    assert np.array_equal(perm[0, 0], p_or)
    assert np.array_equal(C[0, 0], c_or)


@pytest.mark.parametrize("K,iters", [(1, 1), (5, 2), (37, 3), (256, 1)])
def test_cluster_bitexact_warm_shapes(K, iters):
    B, H, N, d = 1, 2, 1024, 128
    w = synth.gen("wan", seed=8, B=B, H=H, N=N, d=d)
    rng = np.random.default_rng(K)
    C0 = rng.standard_normal((B, H, K, d)).astype(np.float32) * 2
    lab, perm, C = _gpu_cluster(w["V"], K, iters, False, C0)
    for h in range(H):
        l_or, p_or, c_or = oracle.kmeans(w["V"][0, h], K, iters, cold=False, C=C0[0, h])
        assert np.array_equal(lab[0, h], l_or)
        assert np.array_equal(perm[0, h], p_or)
        assert np.array_equal(C[0, h], c_or)


def test_cluster_ties_duplicate_centroids():
    """Duplicate centroids and integer data: exact ties must go to the lowest index."""
    B, H, N, d, K = 1, 1, 512, 64, 6
    rng = np.random.default_rng(12)
    V = synth.bf16_bits((rng.integers(-3, 4, (B, H, N, d)) * 0.5).astype(np.float32))
    C0 = (rng.integers(-3, 4, (B, H, K, d)) * 0.5).astype(np.float32)
    C0[0, 0, 4] = C0[0, 0, 1]
    lab, perm, C = _gpu_cluster(V, K, 1, False, C0)
    l_or, p_or, c_or = oracle.kmeans(V[0, 0], K, 1, cold=False, C=C0[0, 0])
    assert np.array_equal(lab[0, 0], l_or)
    assert np.array_equal(perm[0, 0], p_or)
    assert np.array_equal(C[0, 0], c_or)


@pytest.mark.parametrize("d", [64, 128])
def test_cluster_ties_reranked_in_batches(d):
    """90 centroids in identical pairs (2i, 2i+1) and 10 single ones, tokens near them: a
    token near a pair has an exact tie for its best distance and goes through the exact
    re-rank, so every work-group re-ranks about 200 of its tokens, a count that is not a
    multiple of the re-rank's batches (K = 100 is not a multiple of the centroids ranked per
    step either; the last work-group holds 128 tokens). Tokens of a pair must get its even
    index, as the oracle has it."""
    B, H, N, NP, NS = 1, 2, 1152, 45, 10
    K = 2 * NP + NS
    rng = np.random.default_rng(21 + d)
    base = (rng.integers(-6, 7, (B, H, NP + NS, d)) * 0.5).astype(np.float32)
    C0 = np.concatenate([np.repeat(base[:, :, :NP], 2, axis=2), base[:, :, NP:]], axis=2)
    pick = rng.integers(0, NP + NS, (B, H, N))
    noise = (rng.integers(-1, 2, (B, H, N, d)) * 0.5).astype(np.float32)
    noise *= rng.random((B, H, N, d)) < 0.1
    Vf = np.take_along_axis(base, pick[..., None].repeat(d, -1), axis=2) + noise
    V = synth.bf16_bits(Vf)
    lab, perm, C = _gpu_cluster(V, K, 1, False, C0)
    for h in range(H):
        l_or, p_or, c_or = oracle.kmeans(V[0, h], K, 1, cold=False, C=C0[0, h])
        paired = l_or < 2 * NP
        assert np.all(l_or[paired] % 2 == 0) and 0.7 < paired.mean() < 0.9
        assert np.array_equal(lab[0, h], l_or), (h, np.count_nonzero(lab[0, h] != l_or))
        assert np.array_equal(perm[0, h], p_or)
        assert np.array_equal(C[0, h], c_or)


def _gpu_cluster_balanced(V, K, iters, cold, lam, counts, C0=None):
    B, H, N, d = V.shape
    C = torch.zeros((B, H, K, d), dtype=torch.float32, device="cuda") if C0 is None else to_dev(C0)
    cnt = to_dev(np.ascontiguousarray(counts, dtype=np.int32))
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    vc.vc_cluster_balanced(to_dev_bf16(V), K, iters, cold, lam, cnt, C, lab, perm)
    torch.cuda.synchronize()
    return lab.cpu().numpy(), perm.cpu().numpy(), C.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("d,N,K,iters", [(128, 1024, 8, 3), (64, 2560, 37, 2), (128, 3072, 300, 2)])
@pytest.mark.parametrize("kappa", [0.0, 0.01, 0.3, 30.0])
def test_cluster_balanced_bitexact(d, N, K, iters, kappa):
    """Size-penalised k-means, warm start with given sizes, several heads and a ragged last
    work-group; lambda = kappa * J / (N/K) with J the plain mean squared distance, from no
    effect up to the oscillating regime. Labels, perm, centroids and sizes bit-exact."""
    B, H = 1, 2
    w = synth.gen("wan", seed=14, B=B, H=H, N=N, d=d)
    rng = np.random.default_rng(N + K)
    C0 = (rng.standard_normal((B, H, K, d)) * 2).astype(np.float32)
    cnt0 = rng.integers(0, 3 * N // K + 1, (B, H, K)).astype(np.int32)
    lab0, _, _ = oracle.kmeans(w["V"][0, 0], K, 1, cold=False, C=C0[0, 0])
    J = oracle.kmeans_cost(w["V"][0, 0], C0[0, 0], lab0)
    lam = float(np.float32(kappa * J * K / N))
    lab, perm, C, cnt = _gpu_cluster_balanced(w["V"], K, iters, False, lam, cnt0, C0)
    for h in range(H):
        l_or, p_or, c_or, n_or = oracle.kmeans_balanced(w["V"][0, h], K, iters, False, lam, cnt0[0, h], C0[0, h])
        assert np.array_equal(lab[0, h], l_or), (h, np.count_nonzero(lab[0, h] != l_or))
        assert np.array_equal(perm[0, h], p_or)
        assert np.array_equal(C[0, h], c_or)
        assert np.array_equal(cnt[0, h], n_or)


def test_cluster_balanced_lambda_zero_equals_plain():
    w = synth.gen("wan", seed=8, B=1, H=2, N=2048, d=128)
    a = _gpu_cluster(w["V"], 16, 2, True)
    b = _gpu_cluster_balanced(w["V"], 16, 2, True, 0.0, np.full((1, 2, 16), 99, np.int32))
    for x, y in zip(a, b[:3]):
        assert np.array_equal(x, y)
    assert np.array_equal(b[3][0, 0], np.bincount(a[0][0, 0], minlength=16))


def test_cluster_balanced_ties_and_rerank():
    """Integer data, duplicate centroids with equal sizes (exact ties: lowest index) and
    with sizes one apart (the penalty alone decides): exercises the exact re-rank."""
    B, H, N, d, K = 1, 1, 512, 64, 6
    rng = np.random.default_rng(12)
    V = synth.bf16_bits((rng.integers(-3, 4, (B, H, N, d)) * 0.5).astype(np.float32))
    C0 = (rng.integers(-3, 4, (B, H, K, d)) * 0.5).astype(np.float32)
    C0[0, 0, 4] = C0[0, 0, 1]
    C0[0, 0, 5] = C0[0, 0, 2]
    cnt0 = np.array([[[40, 70, 71, 30, 70, 70]]], np.int32)
    for lam in (0.25, 0.0625):
        lab, perm, C, cnt = _gpu_cluster_balanced(V, K, 2, False, lam, cnt0, C0)
        l_or, p_or, c_or, n_or = oracle.kmeans_balanced(V[0, 0], K, 2, False, lam, cnt0[0, 0], C0[0, 0])
        assert np.array_equal(lab[0, 0], l_or)
        assert np.array_equal(perm[0, 0], p_or)
        assert np.array_equal(C[0, 0], c_or)
        assert np.array_equal(cnt[0, 0], n_or)


@pytest.mark.parametrize("d,N,K", [(128, 1024, 8), (64, 2560, 37), (128, 3072, 300)])
def test_cluster_cost_matches_oracle(d, N, K):
    """k-means objective under given (arbitrary) labels and centroids, several heads,
    a ragged last work-group: binary64 sums within 1e-11 of the exact value."""
    B, H = 1, 3
    rng = np.random.default_rng(N + K)
    w = synth.gen("wan", seed=12, B=B, H=H, N=N, d=d)
    C = (rng.standard_normal((B, H, K, d)) * 2).astype(np.float32)
    lab = rng.integers(0, K, (B, H, N)).astype(np.int32)
    cost = torch.empty((B, H), dtype=torch.float64, device="cuda")
    vc.vc_cluster_cost(to_dev_bf16(w["V"]), to_dev(C), to_dev(lab), cost)
    got = cost.cpu().numpy()
    for h in range(H):
        want = oracle.kmeans_cost(w["V"][0, h], C[0, h], lab[0, h])
        assert abs(got[0, h] - want) <= 1e-11 * want, (h, got[0, h], want)


def test_cluster_deterministic():
    w = synth.gen("wan", seed=8, B=1, H=2, N=2048, d=128)
    a = _gpu_cluster(w["V"], 16, 2, True)
    b = _gpu_cluster(w["V"], 16, 2, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------------------ attention
def _gpu_attention(out, N, d, B, H, expcast, restore, dump_block=None, e5m2=False, mx=False):
    O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    flags = (vc.VC_F_EXPCAST | (vc.VC_F_E5M2 if e5m2 else 0)) if expcast else 0
    flags |= vc.VC_F_MXFP4 if mx else 0
    beta = BETA2 if e5m2 else BETA
    if dump_block is None:
        vc.vc_attention(out, O, beta=beta, flags=flags, restore_mean=restore)
        torch.cuda.synchronize()
        return bf16_bits(O), None
    codes = torch.zeros((B, H, N, 128), dtype=torch.uint8, device="cuda")
    vc.vc_attention_dump(out, O, dump_block, codes, beta=beta, flags=flags, restore_mean=restore)
    torch.cuda.synchronize()
    return bf16_bits(O), codes.cpu().numpy()


def _o_f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("path", ["vc", "vsmooth", "plain", "expcast", "vc_e5m2", "expcast_e5m2"])
def test_attention_matches_emulation_tiny(path):
    w = synth.gen("tiny")
    N, d = 1024, 128
    expcast = path.startswith(("vc", "expcast"))
    e5m2 = path.endswith("e5m2")
    vs = path.startswith(("vc", "vsmooth"))
    perm = synth.rand_perm(N, 1) if vs else None
    flags = vc.VC_F_KSMOOTH | (vc.VC_F_VSMOOTH if vs else 0)
    out = gpu_quantize(w["Q"], w["K"], w["V"], None if perm is None else perm[None, None], flags)
    O, _ = _gpu_attention(out, N, d, 1, 1, expcast, vs, e5m2=e5m2)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], perm, flags)
    rows = np.arange(N, dtype=np.int32)
    mode = (oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST) if expcast else oracle.MODE_EXP_THEN_CAST
    O_or = oracle.attention_emul(q_or, rows, beta=BETA2 if e5m2 else BETA, mode=mode, restore_mean=vs)
    err = rel_l2(_o_f64(O[0, 0]), O_or)
    print("[tiny %s] rel-L2 vs emulation %.3e" % (path, err))
    assert err <= (TOL_E5M2 if e5m2 else TOL), err


@pytest.mark.parametrize("e5m2", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [128, 640])
def test_attention_matches_emulation_shapes(d, N, e5m2):
    B, H = 2, 2
    w = synth.gen("wan", seed=6, B=B, H=H, N=N, d=d)
    perm = np.stack([np.stack([synth.rand_perm(N, 4, b, h) for h in range(H)]) for b in range(B)])
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm, FLAGS_ALL)
    O, _ = _gpu_attention(out, N, d, B, H, True, True, e5m2=e5m2)
    rows = np.arange(N, dtype=np.int32)
    mode = oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST
    for b in range(B):
        for h in range(H):
            q_or = oracle.quantize(w["Q"][b, h], w["K"][b, h], w["V"][b, h], perm[b, h], FLAGS_ALL)
            O_or = oracle.attention_emul(q_or, rows, beta=BETA2 if e5m2 else BETA, mode=mode)
            err = rel_l2(_o_f64(O[b, h]), O_or)
            print("[shapes N=%d d=%d %s] (%d,%d) rel-L2 vs emulation %.3e" % (N, d, "e5m2" if e5m2 else "e4m3", b, h, err))
            assert err <= (TOL_E5M2 if e5m2 else TOL), (b, h, err)


@pytest.mark.parametrize("d,N", [(128, 1024), (64, 640)])
@pytest.mark.parametrize("path", ["vsmooth", "vc", "plain"])
def test_attention_mxfp4_matches_emulation(path, d, N):
    """4-bit (MXFP4) value residual on the block-scaled MFMA: exp-then-cast with V-Smooth
    (the pages' 4-bit configuration), ExpCast with V-Smooth, and plain exp-then-cast."""
    expcast = path == "vc"
    vs = path != "plain"
    w = synth.gen("wan", seed=16, B=1, H=1, N=N, d=d)
    perm = synth.rand_perm(N, 3) if vs else None
    flags = vc.VC_F_KSMOOTH | (vc.VC_F_VSMOOTH if vs else 0) | vc.VC_F_MXFP4
    out = gpu_quantize(w["Q"], w["K"], w["V"], None if perm is None else perm[None, None], flags)
    O, _ = _gpu_attention(out, N, d, 1, 1, expcast, vs, mx=True)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], perm, int(flags))
    rows = np.arange(N, dtype=np.int32)
    O_or = oracle.attention_emul(q_or, rows, beta=BETA,
                                 mode=oracle.MODE_EXPCAST if expcast else oracle.MODE_EXP_THEN_CAST, restore_mean=vs)
    err = rel_l2(_o_f64(O[0, 0]), O_or)
    print("[mxfp4 %s d=%d] rel-L2 vs emulation %.3e" % (path, d, err))
    assert err <= TOL, err


def _score_error_band(q_or, rows, blk):
    """Upper bound of |hardware score - exactly rounded score| for each (row, key) of
    block `blk`, from the accumulation model of the gfx950 FP8 MFMA."""
    def split(codes):
        c = codes.astype(np.int64)
        e = (c >> 3) & 15
        m = c & 7
        val = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * np.exp2(e - 7.0))
        val = np.where((c >> 7) == 1, -val, val)
        floor_mag = np.exp2(np.where(e == 0, -6, e - 7).astype(np.float64))
        return val, floor_mag
    qa, qf = split(q_or["Qq"][rows])                  # [R, d]
    kb = q_or["Kq"][blk * 128:(blk + 1) * 128]
    ka, kf = split(kb)                                # [128, d]
    d = qa.shape[1]
    absprod = np.abs(qa)[:, None, :] * np.abs(ka)[None, :, :]            # [R,128,d]
    expo = qf[:, None, :] * kf[None, :, :]                               # 2^(ea+eb)
    grp = expo.reshape(len(rows), 128, d // 8, 8).max(-1)                # per group of 8 K-slots
    return grp.sum(-1) * 2.0 ** -10 + absprod.sum(-1) * 2.0 ** -20


@pytest.mark.parametrize("e5m2", [False, True])
def test_inkernel_expcast_bytes_tiny(e5m2):
    """In-kernel ExpCast bytes (E4M3, or the E5M2 variant) against the emulation: at least
    99 % equal; every other byte differs by one code and its oracle pre-rounding value lies
    within the hardware score-error band of the boundary between the two codes."""
    w = synth.gen("tiny")
    N, d = 1024, 128
    perm = synth.rand_perm(N, 1)
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm[None, None], FLAGS_ALL)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], perm, FLAGS_ALL)
    rows = np.arange(N, dtype=np.int32)
    slope, beta = (4.0, BETA2) if e5m2 else (8.0, BETA)
    mode = oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST
    total, agree = 0, 0
    for blk in (0, 3, 7):
        _, codes = _gpu_attention(out, N, d, 1, 1, True, True, dump_block=blk, e5m2=e5m2)
        _, c_or, m_or = oracle.attention_emul(q_or, rows, beta=beta, mode=mode, dump_block=blk, want_m=True)
        got = codes[0, 0]
        total += got.size
        agree += int((got == c_or).sum())
        bad = np.argwhere(got != c_or)
        if bad.size == 0:
            continue
        assert np.all(np.abs(got.astype(int) - c_or.astype(int))[got != c_or] == 1)
        # oracle pre-rounding value t and its distance to the boundary between the two codes
        band = _score_error_band(q_or, rows, blk)                         # [N,128] in score units
        I = rows // 128
        sig = (q_or["sQ"][I] * q_or["sK"][blk]).astype(np.float32)      # per row
        acc = np.zeros((N, 128))
        qv = oracle.e4m3_decode(q_or["Qq"]).astype(np.float64)
        kv = oracle.e4m3_decode(q_or["Kq"][blk * 128:(blk + 1) * 128]).astype(np.float64)
        acc = (qv @ kv.T).astype(np.float32).astype(np.float64)
        mp = m_or[:, blk].astype(np.float64)
        t = acc * (slope * sig[:, None]) + (np.float64(np.float32(120.0 + np.float32(beta))) - slope * mp[:, None])
        # running-max shift bound: the maximum band over this row's blocks so far, scaled
        dm = np.zeros(N)
        for j in range(blk + 1):
            bj = _score_error_band(q_or, rows, j).max(1)
            dm = np.maximum(dm, bj * (q_or["sQ"][I] * q_or["sK"][j]))
        dt = slope * sig[:, None] * band + slope * dm[:, None] + 1e-4
        for r_, c_ in bad:
            lo = min(int(got[r_, c_]), int(c_or[r_, c_]))
            boundary = lo + 0.5
            assert abs(t[r_, c_] - boundary) <= dt[r_, c_], (blk, r_, c_, t[r_, c_], dt[r_, c_])
    print("[in-kernel %s bytes] agreement %.5f" % ("e5m2" if e5m2 else "e4m3", agree / total))
    assert agree / total >= 0.99, agree / total


# ------------------------------------------------------------------ properties at any size
def test_perm_is_stable_sort_of_labels():
    w = synth.gen("wan", seed=13, B=1, H=3, N=4096, d=128)
    lab, perm, _ = _gpu_cluster(w["V"], 32, 2, True)
    for h in range(3):
        assert np.array_equal(np.sort(perm[0, h]), np.arange(4096))
        assert np.array_equal(perm[0, h], np.argsort(lab[0, h], kind="stable"))


@pytest.mark.parametrize("e5m2", [False, True])
def test_attention_huge_scores_clamped_path(e5m2):
    """Scores whose running maximum exceeds 2^16 in log2 units take the kernel's clamped
    ExpCast branch; output and dumped bytes must still match the emulation."""
    beta = BETA2 if e5m2 else BETA
    mode = oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST
    N, d = 512, 128
    rng = np.random.default_rng(31)
    Q = synth.bf16_bits((rng.standard_normal((1, 1, N, d)) * 300).astype(np.float32))
    K = synth.bf16_bits((rng.standard_normal((1, 1, N, d)) * 300).astype(np.float32))
    V = synth.bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    out = gpu_quantize(Q, K, V, None, vc.VC_F_KSMOOTH)
    q_or = oracle.quantize(Q[0, 0], K[0, 0], V[0, 0], None, oracle.FLAG_KSMOOTH)
    rows = np.arange(N, dtype=np.int32)
    _, c_or, m_or = oracle.attention_emul(q_or, rows, beta=beta, mode=mode, dump_block=2, want_m=True)
    assert np.abs(m_or).max() >= 65536.0
    O, codes = _gpu_attention(out, N, d, 1, 1, True, False, dump_block=2, e5m2=e5m2)
    O_or = oracle.attention_emul(q_or, rows, beta=beta, mode=mode, restore_mean=False)
    assert rel_l2(_o_f64(O[0, 0]), O_or) <= (TOL_E5M2 if e5m2 else TOL)
    agree = np.mean(codes[0, 0] == c_or)
    assert agree >= 0.99, agree
