"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: ExpCast bytes (the kernel's byte sequence elementwise, and the bytes inside the
attention loop), quantiser outputs (codes, scales, means), k-means labels / permutation /
centroids, and the FP8 matrix core's scores against the oracle's model of them. The oracle
takes every score in the matrix core's precision (oracle.attention_emul(score="gfx950")), the
precision the kernel decides its bytes in, and rounds the output to bfloat16; the attention
output must then lie within relative L2 2e-3 of that emulation (the exact-score figure is
printed beside it).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402

vc = pytest.importorskip("bit_attention_video_online_amd")
from tests.gpu_util import (bf16_bits, emul, gpu_quantize, mu_pack_expected, mx_unpack, rel_l2, to_dev,  # noqa: E402
                            to_dev_bf16, vq_rowmajor)

BETA = oracle.BETA_E4M3
BETA2 = oracle.BETA_E5M2
# Output tolerance: relative L2 2e-3 against the emulation, for every probability format (the
# bytes themselves are bit-exact, so what remains is accumulation order, the row-sum and mean
# operands of the matrix core and the output rounding).
TOL = 2e-3
FLAGS_ALL = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH


def _ok():
    return torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not _ok():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ ExpCast function
def _expcast_inputs(rng, n):
    acc = (rng.standard_normal(n) * np.exp2(rng.integers(-6, 14, n))).astype(np.float32)
    s8 = (8.0 * np.exp2(rng.uniform(-16, -2, n))).astype(np.float32)
    mprime = (rng.uniform(-50, 50, n)).astype(np.float32)
    bias = (np.float32(np.float32(120.0) + np.float32(BETA)) - np.float32(8.0) * mprime).astype(np.float32)
    return acc, s8, bias


def test_expcast_function_bitexact_clamped_path():
    """The kernel's byte sequence with the per-byte clamp, on arbitrary inputs, ties and clamp
    edges: every byte equals the oracle's clamp(rne(fma(acc, s, b)), 0, 120)."""
    rng = np.random.default_rng(7)
    acc, s8, bias = _expcast_inputs(rng, 1 << 20)
    k = rng.integers(-3, 124, 4096).astype(np.float32)
    acc = np.concatenate([acc, k + np.float32(0.5), k, np.float32([120.5, 121.5, -0.5, -0.51, 0.49, 119.65, 1e9, -1e9])])
    s8 = np.concatenate([s8, np.ones(2 * 4096 + 8, np.float32)])
    bias = np.concatenate([bias, np.zeros(2 * 4096 + 8, np.float32)])
    want = oracle.expcast(acc, s8, bias)
    out = torch.empty(acc.size, dtype=torch.uint8, device="cuda")
    vc.vc_debug_expcast(to_dev(acc), to_dev(s8), to_dev(bias), out)
    got = out.cpu().numpy()
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]


def test_expcast_function_bitexact_unclamped_path():
    """The kernel's byte sequence without the clamp (its usual path), on the inputs it takes it
    for: scores below the running maximum m' (|m'| < 2^16) with beta <= 0.35. Every byte equals
    the oracle's; a ragged length exercises the packing of the last dword."""
    rng = np.random.default_rng(8)
    n = (1 << 20) + 3
    sigma = np.exp2(rng.uniform(-16, -2, n)).astype(np.float32)
    mprime = rng.uniform(-60000, 60000, n).astype(np.float32)
    u = -rng.exponential(6.0, n)                                     # log2-domain score minus m'
    acc = ((mprime.astype(np.float64) + u) / sigma).astype(np.float32)
    mprime = np.maximum(mprime, (sigma * acc).astype(np.float32))   # m' >= fl32(sigma acc)
    beta = rng.uniform(-2.0, 0.35, n).astype(np.float32)
    C0 = (np.float32(120.0) + beta).astype(np.float32)
    s8 = (np.float32(8.0) * sigma).astype(np.float32)
    bias = (C0 - np.float32(8.0) * mprime).astype(np.float32)
    want = oracle.expcast(acc, s8, bias)
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    vc.vc_debug_expcast(to_dev(acc), to_dev(s8), to_dev(bias), out, clamp=False)
    got = out.cpu().numpy()
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]
    assert want.max() <= 120 and (want == 120).any() and (want == 0).any()


def _gauss_codes(rng, shape, t_dof=None):
    x = rng.standard_normal(shape) if t_dof is None else rng.standard_t(t_dof, shape)
    return oracle.e4m3_encode((x * 448.0 / np.abs(x).max(axis=(-2, -1), keepdims=True)).astype(np.float32))


def test_mfma_tiles_match_the_oracles_score_model():
    """The FP8 matrix-core instruction of the kernel against the oracle's model of its
    accumulation (oracle.mfma_f8_dot64), bit for bit: tiles of Gaussian and heavy-tailed codes
    scaled to the E4M3 range (the quantised Q/K the scores come from), one instruction and two
    chained through the accumulator as for d = 128; one product with or without C; two products
    with C = 0. On operands with one product of random exponent in every group beside a large C,
    and on two products beside a C, the model is not exact; that agreement is printed."""
    rng = np.random.default_rng(40)
    n = 256
    A0, B0, A1, B1 = (_gauss_codes(rng, (n, 32, 64), None if i % 2 == 0 else 4) for i in range(4))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    Z = torch.zeros((n, 32, 32), dtype=torch.float32, device="cuda")
    D1 = torch.empty_like(Z)
    D2 = torch.empty_like(Z)
    vc.vc_debug_mfma_f8(dev(A0), dev(B0), Z, D1)
    vc.vc_debug_mfma_f8(dev(A1), dev(B1), D1, D2)
    d1, d2 = D1.cpu().numpy(), D2.cpu().numpy()
    pair = lambda A, B: (np.repeat(A[:, :, None, :], 32, 2), np.repeat(B[:, None, :, :], 32, 1))
    m1 = oracle.mfma_f8_dot64(*pair(A0, B0), np.zeros((n, 32, 32), np.float32))
    m2 = oracle.mfma_f8_dot64(*pair(A1, B1), m1)
    assert np.array_equal(d1, m1), np.count_nonzero(d1 != m1)
    assert np.array_equal(d2, m2), np.count_nonzero(d2 != m2)
    # sparse operands, random codes over the whole E4M3 range: even rows one nonzero slot and a C
    # that is zero or random; odd rows two nonzero slots (same group or not) and C = 0
    good = np.array([c for c in range(256) if (c & 0x7F) not in (0, 0x7F)], np.uint8)
    A = np.zeros((n, 32, 64), np.uint8)
    for t in range(n):
        for r in range(32):
            A[t, r, rng.choice(64, 1 + (r & 1), replace=False)] = rng.choice(good, 1 + (r & 1))
    B = rng.choice(good, (n, 32, 64))
    C = np.where(rng.random((n, 32, 32)) < 0.5, 0.0,
                 rng.standard_normal((n, 32, 32)) * np.exp2(rng.integers(-20, 18, (n, 32, 32)))).astype(np.float32)
    C[:, 1::2, :] = 0.0
    D = torch.empty_like(Z)
    vc.vc_debug_mfma_f8(dev(A), dev(B), dev(C), D)
    got, want = D.cpu().numpy(), oracle.mfma_f8_dot64(*pair(A, B), C)
    for t, r, c in np.argwhere(got != want)[:8]:
        ks = np.nonzero(A[t, r])[0]
        print("[mfma model] mismatch tile %d row %d col %d: slots %s a %s b %s C %r got %r model %r"
              % (t, r, c, ks.tolist(), [hex(x) for x in A[t, r, ks]], [hex(x) for x in B[t, c, ks]],
                 float(C[t, r, c]), float(got[t, r, c]), float(want[t, r, c])))
    assert np.array_equal(got, want), np.count_nonzero(got != want)
    # adversarial: every group one product of random exponent, C of comparable size (not modelled)
    A = np.zeros((n, 32, 64), np.uint8)
    for g in range(8):
        A[np.arange(n)[:, None], np.arange(32)[None, :], 8 * g + rng.integers(0, 8, (n, 32))] = rng.choice(good, (n, 32))
    C = (rng.choice([-1, 1], (n, 32, 32)) * np.exp2(rng.integers(-6, 18, (n, 32, 32)))).astype(np.float32)
    vc.vc_debug_mfma_f8(dev(A), dev(B), dev(C), D)
    agree = np.mean(D.cpu().numpy() == oracle.mfma_f8_dot64(*pair(A, B), C))
    A2 = np.zeros((n, 32, 64), np.uint8)
    for t in range(n):
        for r in range(32):
            A2[t, r, rng.choice(64, 2, replace=False)] = rng.choice(good, 2)
    C2 = (rng.standard_normal((n, 32, 32)) * np.exp2(rng.integers(-20, 18, (n, 32, 32)))).astype(np.float32)
    vc.vc_debug_mfma_f8(dev(A2), dev(B), dev(C2), D)
    agree2 = np.mean(D.cpu().numpy() == oracle.mfma_f8_dot64(*pair(A2, B), C2))
    print("[mfma model] outputs reproduced: one product per group beside a large C %.4f; two products "
          "beside a C %.4f" % (agree, agree2))


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
    O_or = emul(q_or, rows, beta=BETA2 if e5m2 else BETA, mode=oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST)
    err = rel_l2(_o_f64(O[0, 0]), O_or)
    print("[rope+hadamard %s] rel-L2 vs emulation %.3e" % ("e5m2" if e5m2 else "e4m3", err))
    assert err <= (TOL), err


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
@pytest.mark.parametrize("m", [2, 3])
def test_cluster_ties_reranked_in_batches(d, m):
    """Centroids in groups of m identical copies (45 pairs, or 30 triples) plus 10 single ones,
    tokens near them: a token near a group has an exact tie for its best distance. With
    pairs, the third smallest distance is clearly larger and the two tied centroids' exact
    distances decide; with triples, the three-way tie goes through the batched exact re-rank,
    so every work-group re-ranks about 200 of its tokens, a count that is not a multiple of
    the re-rank's batches (K is not a multiple of the centroids ranked per step either; the
    last work-group holds 128 tokens). Tokens of a group must get its first index, as the
    oracle has it."""
    B, H, N, NS = 1, 2, 1152, 10
    NG = 90 // m
    K = m * NG + NS
    rng = np.random.default_rng(21 + d + 100 * m)
    base = (rng.integers(-6, 7, (B, H, NG + NS, d)) * 0.5).astype(np.float32)
    C0 = np.concatenate([np.repeat(base[:, :, :NG], m, axis=2), base[:, :, NG:]], axis=2)
    pick = rng.integers(0, NG + NS, (B, H, N))
    noise = (rng.integers(-1, 2, (B, H, N, d)) * 0.5).astype(np.float32)
    noise *= rng.random((B, H, N, d)) < 0.1
    Vf = np.take_along_axis(base, pick[..., None].repeat(d, -1), axis=2) + noise
    V = synth.bf16_bits(Vf)
    lab, perm, C = _gpu_cluster(V, K, 1, False, C0)
    for h in range(H):
        l_or, p_or, c_or = oracle.kmeans(V[0, h], K, 1, cold=False, C=C0[0, h])
        grouped = l_or < m * NG
        assert np.all(l_or[grouped] % m == 0) and 0.7 < grouped.mean() < 0.95
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
def _gpu_attention(out, N, d, B, H, expcast, restore, dump_block=None, e5m2=False, mx=False, beta=None):
    O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    flags = (vc.VC_F_EXPCAST | (vc.VC_F_E5M2 if e5m2 else 0)) if expcast else 0
    flags |= vc.VC_F_MXFP4 if mx else 0
    beta = (BETA2 if e5m2 else BETA) if beta is None else beta
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
    O_or = emul(q_or, rows, beta=BETA2 if e5m2 else BETA, mode=mode, restore_mean=vs)
    err = rel_l2(_o_f64(O[0, 0]), O_or)
    err_x = rel_l2(_o_f64(O[0, 0]), oracle.attention_emul(q_or, rows, beta=BETA2 if e5m2 else BETA, mode=mode,
                                                        restore_mean=vs))
    print("[tiny %s] rel-L2 vs emulation %.3e (exactly rounded scores, unrounded output: %.3e)" % (path, err, err_x))
    assert err <= (TOL), err


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
            O_or = emul(q_or, rows, beta=BETA2 if e5m2 else BETA, mode=mode)
            err = rel_l2(_o_f64(O[b, h]), O_or)
            print("[shapes N=%d d=%d %s] (%d,%d) rel-L2 vs emulation %.3e" % (N, d, "e5m2" if e5m2 else "e4m3", b, h, err))
            assert err <= (TOL), (b, h, err)


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
    O_or = emul(q_or, rows, beta=BETA, mode=oracle.MODE_EXPCAST if expcast else oracle.MODE_EXP_THEN_CAST,
                restore_mean=vs)
    err = rel_l2(_o_f64(O[0, 0]), O_or)
    print("[mxfp4 %s d=%d] rel-L2 vs emulation %.3e" % (path, d, err))
    assert err <= TOL, err


@pytest.mark.parametrize("e5m2", [False, True])
def test_inkernel_expcast_bytes_bitexact_tiny(e5m2):
    """Probability bytes inside the attention loop (E4M3, and the E5M2 variant), dumped for key
    blocks 0, 3 and 7 of every query row: all bytes equal the emulation's, whose scores are
    taken in the matrix core's precision; so is the output within the tolerance."""
    w = synth.gen("tiny")
    N, d = 1024, 128
    perm = synth.rand_perm(N, 1)
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm[None, None], FLAGS_ALL)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], perm, FLAGS_ALL)
    rows = np.arange(N, dtype=np.int32)
    beta = BETA2 if e5m2 else BETA
    mode = oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST
    exact_agree = []
    for blk in (0, 3, 7):
        O, codes = _gpu_attention(out, N, d, 1, 1, True, True, dump_block=blk, e5m2=e5m2)
        O_or, c_or = emul(q_or, rows, beta=beta, mode=mode, dump_block=blk)
        assert np.array_equal(codes[0, 0], c_or), (blk, np.count_nonzero(codes[0, 0] != c_or))
        assert rel_l2(_o_f64(O[0, 0]), O_or) <= TOL
        _, c_x = oracle.attention_emul(q_or, rows, beta=beta, mode=mode, dump_block=blk)
        exact_agree.append(np.mean(codes[0, 0] == c_x))
    print("[in-kernel %s bytes] bit-exact; agreement with exactly rounded scores would be %s"
          % ("e5m2" if e5m2 else "e4m3", ["%.5f" % a for a in exact_agree]))


@pytest.mark.parametrize("d,mx", [(64, False), (128, True), (64, True)])
def test_inkernel_expcast_bytes_bitexact_d64_and_mxfp4(d, mx):
    """The same byte check for the other kernel instantiations that ship ExpCast: d = 64 (one
    matrix-core instruction per score, C = 0) and the 4-bit (MXFP4) value residual, whose V
    tiles and PV instruction differ but whose scores and bytes must not; blocks 0, 3 and 7."""
    N = 1024
    w = synth.gen("tiny", d=d)
    perm = synth.rand_perm(N, 2)
    fl = FLAGS_ALL | (vc.VC_F_MXFP4 if mx else 0)
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm[None, None], fl)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], perm,
                           oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH | (oracle.FLAG_MXFP4 if mx else 0))
    rows = np.arange(N, dtype=np.int32)
    for blk in (0, 3, 7):
        O, codes = _gpu_attention(out, N, d, 1, 1, True, True, dump_block=blk, mx=mx)
        O_or, c_or = emul(q_or, rows, beta=BETA, mode=oracle.MODE_EXPCAST, dump_block=blk)
        assert np.array_equal(codes[0, 0], c_or), (blk, np.count_nonzero(codes[0, 0] != c_or))
        assert rel_l2(_o_f64(O[0, 0]), O_or) <= TOL, blk


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
    O_or, c_or, m_or = emul(q_or, rows, beta=beta, mode=mode, restore_mean=False, dump_block=2, want_m=True)
    assert np.abs(m_or).max() >= 65536.0
    O, codes = _gpu_attention(out, N, d, 1, 1, True, False, dump_block=2, e5m2=e5m2)
    assert rel_l2(_o_f64(O[0, 0]), O_or) <= TOL
    assert np.array_equal(codes[0, 0], c_or), np.count_nonzero(codes[0, 0] != c_or)


@pytest.mark.parametrize("e5m2,beta", [(False, 1.0), (False, 0.45), (True, 4.0)])
def test_attention_positive_beta_clamps_codes(e5m2, beta):
    """A positive offset moves the row maximum's byte above 120 before the clamp: fl32(120 +
    beta) > 120 must take the clamped path, so every byte stays in [0, 120] (E4M3: 121..126
    would be larger probabilities, 127 NaN; E5M2: 124 is infinity) and equals the emulation's."""
    w = synth.gen("wan", seed=17, B=1, H=1, N=512, d=128)
    N, d = 512, 128
    mode = oracle.MODE_EXPCAST_E5M2 if e5m2 else oracle.MODE_EXPCAST
    out = gpu_quantize(w["Q"], w["K"], w["V"], None, vc.VC_F_KSMOOTH)
    q_or = oracle.quantize(w["Q"][0, 0], w["K"][0, 0], w["V"][0, 0], None, oracle.FLAG_KSMOOTH)
    rows = np.arange(N, dtype=np.int32)
    for blk in (0, 3):
        O, codes = _gpu_attention(out, N, d, 1, 1, True, False, dump_block=blk, e5m2=e5m2, beta=beta)
        O_or, c_or = emul(q_or, rows, beta=beta, mode=mode, restore_mean=False, dump_block=blk)
        assert c_or.max() <= 120 and (blk > 0 or c_or.max() == 120)
        assert np.array_equal(codes[0, 0], c_or), np.count_nonzero(codes[0, 0] != c_or)
        assert np.isfinite(_o_f64(O[0, 0])).all()
        assert rel_l2(_o_f64(O[0, 0]), O_or) <= TOL


@pytest.mark.parametrize("d,N,H", [(128, 1152, 2), (128, 2176, 1), (64, 1152, 2)])
def test_attention_one_block_last_chunk(d, N, H):
    """N/128 = 8c + 1 key blocks: the mean operand of the last chunk (one key block) is not
    copied inside the loop and is fetched after it; every row of every head against the
    emulation, with the VC path's mean restoration on."""
    B = 1
    w = synth.gen("wan", seed=19, B=B, H=H, N=N, d=d)
    perm = np.stack([np.stack([synth.rand_perm(N, 23, b, h) for h in range(H)]) for b in range(B)])
    out = gpu_quantize(w["Q"], w["K"], w["V"], perm, FLAGS_ALL)
    O, _ = _gpu_attention(out, N, d, B, H, True, True)
    rows = np.arange(N, dtype=np.int32)
    for h in range(H):
        q_or = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], perm[0, h], FLAGS_ALL)
        err = rel_l2(_o_f64(O[0, h]), emul(q_or, rows, beta=BETA, mode=oracle.MODE_EXPCAST))
        print("[last chunk N=%d d=%d] head %d rel-L2 %.3e" % (N, d, h, err))
        assert err <= TOL, (h, err)


def test_attention_d64_long_sequence_sampled_rows():
    """d = 64 at N = 32,768 (the head-size sweep's d = 64 point; 256 key blocks, so 32 flushes
    of the mean operand): k-means permutation from the GPU, quantiser bit-exact against the
    oracle, output on 64 sampled rows of two heads within the tolerance."""
    B, H, N, d = 1, 2, 32768, 64
    w = synth.gen("sweep", seed=44, B=B, H=H, N=N, d=d)
    Vd = to_dev_bf16(w["V"])
    C = torch.zeros((B, H, N // 128, d), dtype=torch.float32, device="cuda")
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    vc.vc_cluster(Vd, N // 128, 2, True, C, lab, perm)
    pm = perm.cpu().numpy()
    out = gpu_quantize(w["Q"], w["K"], w["V"], pm, FLAGS_ALL)
    O, _ = _gpu_attention(out, N, d, B, H, True, True)
    rng = np.random.default_rng(64)
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    for h in range(H):
        q_or = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], pm[0, h], FLAGS_ALL)
        for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu_scaled"):
            assert np.array_equal(g[k][0, h], q_or[k]), (h, k)
        rows = np.sort(np.concatenate([[0, N - 1], rng.choice(N, 62, replace=False)])).astype(np.int32)
        err = rel_l2(_o_f64(O[0, h][rows]), emul(q_or, rows, beta=BETA, mode=oracle.MODE_EXPCAST))
        print("[d=64 N=32768] head %d rel-L2 %.3e" % (h, err))
        assert err <= TOL, (h, err)


@pytest.mark.parametrize("d,N,K", [(128, 1024, 8), (64, 2560, 37), (128, 3072, 300)])
@pytest.mark.parametrize("decay,assign", [(0.0, True), (0.5, True), (1.0, False), (0.9, False)])
def test_cluster_incremental_bitexact(d, N, K, decay, assign):
    """Cross-step incremental centroid update, two steps in a row (the second on drifted
    values, carrying the first step's centroids and masses): centroids, masses, labels and
    permutation bit-exact against the oracle on two heads, ragged last work-group included."""
    B, H = 1, 2
    w = synth.gen("wan", seed=33, B=B, H=H, N=N, d=d)
    V1 = w["V"]
    V2 = np.stack([np.stack([synth.drift(w["V"][0, h], 33, 0, h, 1) for h in range(H)])])
    rng = np.random.default_rng(N + K)
    C = (rng.standard_normal((B, H, K, d)) * 2).astype(np.float32)
    M = rng.uniform(0, 3 * N / K, (B, H, K)).astype(np.float32)
    M[0, :, :3] = 0.0                                                    # clusters with no history
    lab = rng.integers(0, K, (B, H, N)).astype(np.int32)
    Cd, Md, ld = to_dev(C), to_dev(M), to_dev(lab)
    pd = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    oc, om, ol = C.copy(), M.copy(), lab.copy()
    for step, V in enumerate((V1, V2)):
        vc.vc_cluster_incremental(to_dev_bf16(V), decay, assign, Cd, Md, ld, pd)
        torch.cuda.synchronize()
        for h in range(H):
            l_or, p_or, c_or, m_or = oracle.kmeans_incremental(V[0, h], oc[0, h], om[0, h], decay, assign,
                                                               labels=ol[0, h])
            oc[0, h], om[0, h], ol[0, h] = c_or, m_or, l_or
            assert np.array_equal(ld.cpu().numpy()[0, h], l_or), (step, h)
            assert np.array_equal(pd.cpu().numpy()[0, h], p_or), (step, h)
            assert np.array_equal(Cd.cpu().numpy()[0, h], c_or), (step, h)
            assert np.array_equal(Md.cpu().numpy()[0, h], m_or), (step, h)


def _span_reference(x64: np.ndarray):
    """(largest floor(log2|x|), smallest exponent of a lowest set significand bit) over the
    nonzero finite values, from frexp on binary64 (exact for bf16 and binary32 values)."""
    v = np.abs(x64[np.isfinite(x64) & (x64 != 0)])
    if v.size == 0:
        return (-(2 ** 31), 2 ** 31 - 1)
    m, e = np.frexp(v)
    M = (m * 2.0 ** 53).astype(np.uint64)           # exact: at most 24 significant bits
    tz = np.zeros(M.shape, np.int64)
    r = M.copy()
    while True:
        odd = (r & np.uint64(1)) == 1
        if odd.all():
            break
        tz += ~odd
        r = np.where(odd, r, r >> np.uint64(1))
    return (int((e - 1).max()), int((e - 53 + tz).min()))


def test_exponent_span_matches_reference():
    """vc_exponent_span on bf16 and binary32 tensors (and binary32 read as bf16) against an
    independent frexp computation: random values over a wide exponent range, subnormals,
    signed zeros, infinities and NaNs (ignored), one all-zero head."""
    rng = np.random.default_rng(61)
    B, H, R, d = 2, 3, 70, 24
    x = (rng.standard_normal((B, H, R, d)) * np.exp2(rng.integers(-40, 40, (B, H, R, d)))).astype(np.float32)
    x[0, 1] = 0.0
    x[0, 1, 3, 3] = -0.0
    x[1, 0, 0, :4] = [np.float32(1e-40), np.float32(-3e-45), np.inf, np.nan]   # binary32 subnormals, specials
    x[1, 2, 5, 5] = np.float32(3.0e38)
    xb = synth.bf16_bits(np.nan_to_num(x, nan=0.0, posinf=0.0))
    xb[1, 1, 0, 0] = 0x0001                                                    # smallest bf16 subnormal
    xb[1, 1, 0, 1] = 0x7F80                                                    # bf16 infinity: ignored
    got_b = vc.vc_exponent_span(to_dev_bf16(xb)).cpu().numpy()
    got_f = vc.vc_exponent_span(to_dev(x)).cpu().numpy()
    got_r = vc.vc_exponent_span(to_dev(x), as_bf16=True).cpu().numpy()
    xr = synth.bf16_to_f32(synth.bf16_bits(np.nan_to_num(x, nan=0.0, posinf=0.0))).astype(np.float64)
    for b in range(B):
        for h in range(H):
            assert tuple(got_b[b, h]) == _span_reference(synth.bf16_to_f32(xb[b, h]).astype(np.float64)), (b, h)
            assert tuple(got_f[b, h]) == _span_reference(x[b, h].astype(np.float64)), (b, h)
            assert tuple(got_r[b, h]) == _span_reference(xr[b, h]), (b, h)
    assert tuple(got_b[0, 1]) == (-(2 ** 31), 2 ** 31 - 1)


def test_exponent_span_of_the_video_workload_heads():
    """The checker on Wan-shaped heads (V, keys, and the bf16 centroids after k-means): the
    values must equal the reference, and these heads lie inside the exactness conditions of
    include/vc.h (sums of N terms: span <= 103 - 2 ceil(log2 N); distances: span <= 50 - log2 d,
    43 at d = 128)."""
    N, d, K = 70400, 128, 550
    hs = [synth.gen_head("wan", 2, 0, h, N, d) for h in (0, 23)]
    V = np.stack([w["V"] for w in hs])[None]
    Kt = np.stack([w["K"] for w in hs])[None]
    lab, perm, C = _gpu_cluster(V, K, 2, True)
    sv = vc.vc_exponent_span(to_dev_bf16(V)).cpu().numpy()[0]
    sk = vc.vc_exponent_span(to_dev_bf16(Kt)).cpu().numpy()[0]
    sc = vc.vc_exponent_span(to_dev(C), as_bf16=True).cpu().numpy()[0]
    lim_sum = 103 - 2 * int(np.ceil(np.log2(N)))
    for i in range(2):
        assert tuple(sv[i]) == _span_reference(synth.bf16_to_f32(V[0, i]).astype(np.float64))
        assert tuple(sc[i]) == _span_reference(synth.bf16_to_f32(synth.bf16_bits(C[0, i])).astype(np.float64))
        dist_span = max(sv[i][0], sc[i][0]) - min(sv[i][1], sc[i][1])
        print("[span] head %d: V (E %d, q %d, span %d), K span %d, V with bf16 centroids span %d; sums exact "
              "up to %d: V %s, K %s; distances exact up to 43: %s"
              % (i, sv[i][0], sv[i][1], sv[i][0] - sv[i][1], sk[i][0] - sk[i][1], dist_span, lim_sum,
                 sv[i][0] - sv[i][1] <= lim_sum, sk[i][0] - sk[i][1] <= lim_sum, dist_span <= 43), flush=True)
        assert sv[i][0] - sv[i][1] <= lim_sum and sk[i][0] - sk[i][1] <= lim_sum and dist_span <= 43
