"""GPU parity beyond binary64: the k-means update, the incremental update, the quantiser's
block and key means and the k-means assignment on constructed inputs whose exact results
depend on bits far below binary64 resolution (tests/_wide_span.py; a plain binary64 running
sum gets a large share of them wrong). Every output must equal the oracle's bit for bit and
the constructed exact results."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from tests import _wide_span as ws  # noqa: E402

vc = pytest.importorskip("bit_attention_video_online_amd")
from tests.gpu_util import bf16_bits, gpu_quantize, to_dev, to_dev_bf16, vq_rowmajor  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _clustered_head(rng, d, sizes, columns):
    """len(sizes) clusters, cluster g of sizes[g] tokens: channel g holds 64 for the tokens of
    cluster g (identity channels 0..K-1), the other channels take columns(rng, n, d - K) per
    cluster. Returns (V float64 [sum(sizes), d], labels, per-cluster expected values of the
    other channels)."""
    K = len(sizes)
    V = np.zeros((sum(sizes), d))
    lab = rng.permutation(np.repeat(np.arange(K), sizes)).astype(np.int32)
    exp = []
    for g in range(K):
        X, e = columns(rng, sizes[g], d - K)
        rows = np.flatnonzero(lab == g)
        V[rows, g] = 64.0
        V[rows, K:] = X
        exp.append(np.array(e, np.float32))
    return V, lab, exp


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("sizes", [(256, 256, 256, 256), (200, 312, 97, 415)])
def test_cluster_means_beyond_binary64(d, sizes):
    """vc_cluster, one warm iteration from the identity centroids: labels, perm and centroids
    against the oracle, centroids against the exact means rounded once; cluster sizes powers of
    two (the quotient is exact before its rounding) and not (it is not)."""
    B, H, K = 1, 2, len(sizes)
    N = sum(sizes)
    rng = np.random.default_rng(70 + d + sizes[1])
    heads = [_clustered_head(rng, d, sizes, lambda r, m, c: ws.mean_columns(r, m, c, "f32")[::2]) for _ in range(H)]
    V = np.stack([synth.bf16_bits(h[0].astype(np.float32)) for h in heads])[None]
    C0 = np.zeros((B, H, K, d), np.float32)
    for g in range(K):
        C0[..., g, g] = 64.0
    C = to_dev(C0)
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty_like(lab)
    vc.vc_cluster(to_dev_bf16(V), K, 1, False, C, lab, perm)
    torch.cuda.synchronize()
    Cg, lg, pg = C.cpu().numpy(), lab.cpu().numpy(), perm.cpu().numpy()
    for h in range(H):
        l_or, p_or, c_or = oracle.kmeans(V[0, h], K, 1, cold=False, C=C0[0, h])
        assert np.array_equal(l_or, heads[h][1])
        assert np.array_equal(lg[0, h], l_or), h
        assert np.array_equal(pg[0, h], p_or), h
        assert np.array_equal(Cg[0, h], c_or), (h, np.count_nonzero(Cg[0, h] != c_or))
        for g in range(K):
            assert np.array_equal(Cg[0, h, g, K:], heads[h][2][g]), (h, g)


@pytest.mark.parametrize("d", [64, 128])
def test_cluster_incremental_beyond_binary64(d):
    """vc_cluster_incremental with decay 0 and given labels: C = fl32(fl64(exact sum) / n)
    where the exact sum sits next to a binary64 tie."""
    B, H, K, n = 1, 2, 4, 256
    rng = np.random.default_rng(80 + d)
    heads = [_clustered_head(rng, d, (n,) * K, ws.f64_tie_columns) for _ in range(H)]
    V = np.stack([synth.bf16_bits(h[0].astype(np.float32)) for h in heads])[None]
    lab0 = np.stack([h[1] for h in heads])[None]
    C0 = rng.standard_normal((B, H, K, d)).astype(np.float32)
    M0 = np.full((B, H, K), 9.0, np.float32)
    Cd, Md, ld = to_dev(C0), to_dev(M0), to_dev(lab0)
    pd = torch.empty_like(ld)
    vc.vc_cluster_incremental(to_dev_bf16(V), 0.0, False, Cd, Md, ld, pd)
    torch.cuda.synchronize()
    Cg, Mg = Cd.cpu().numpy(), Md.cpu().numpy()
    for h in range(H):
        l_or, p_or, c_or, m_or = oracle.kmeans_incremental(V[0, h], C0[0, h], M0[0, h], 0.0, False, labels=lab0[0, h])
        assert np.array_equal(pd.cpu().numpy()[0, h], p_or), h
        assert np.array_equal(Cg[0, h], c_or), (h, np.count_nonzero(Cg[0, h] != c_or))
        assert np.array_equal(Mg[0, h], m_or), h
        for g in range(K):
            assert np.array_equal(Cg[0, h, g, K:], heads[h][2][g]), (h, g)


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_means_beyond_binary64(d):
    """vc_quantize with K and V smoothing on permuted keys: block means (bf16 of the exact
    mean of each 128-token block of V') and the key mean (fl32 of the exact mean over the
    sequence) next to rounding ties. The largest smoothed key of block b of K' is 3 - kbar[b]
    (a key of value 3 on channel b), so the key scale sK[b] shows kbar[b]; every output
    against the oracle, bit for bit."""
    B, H, N = 1, 2, 1024
    nb = N // 128
    rng = np.random.default_rng(90 + d)
    Qs, Ks, Vs, perms, mus, kbars, kexact = [], [], [], [], [], [], []
    for h in range(H):
        Vp = np.zeros((N, d))
        mu = np.zeros((nb, d), np.int64)
        for b in range(nb):
            X, _, r = ws.mean_columns(rng, 128, d, "bf16")
            Vp[128 * b:128 * (b + 1)] = X
            mu[b] = r
        perm = synth.rand_perm(N, 91, 0, h)
        V = np.zeros_like(Vp)
        V[perm] = Vp
        Kx, ke, kb = ws.mean_columns(rng, N, d, "f32", small=True)
        for b in range(nb):  # a key of value 3 in block b of K' = K[perm], channel b (column sum kept)
            rows = perm[128 * b:128 * (b + 1)]
            inb = rows[Kx[rows, b] == 2.0]
            out = np.setdiff1d(np.flatnonzero(Kx[:, b] == 2.0), rows)
            Kx[inb[0], b], Kx[out[0], b] = 3.0, 1.0
        Qs.append(synth.gen_head("wan", 92, 0, h, N, d)["Q"])
        Ks.append(synth.bf16_bits(Kx.astype(np.float32)))
        Vs.append(synth.bf16_bits(V.astype(np.float32)))
        perms.append(perm)
        mus.append(mu)
        kbars.append(np.array(kb, np.float32))
        kexact.append(ke)
    Q, K, V, P = (np.stack(x)[None] for x in (Qs, Ks, Vs, perms))
    flags = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH
    out = gpu_quantize(Q, K, V, P, flags)
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    for h in range(H):
        q = oracle.quantize(Q[0, h], K[0, h], V[0, h], P[0, h], int(flags))
        assert np.array_equal(q["mu"].astype(np.int64), mus[h])
        assert np.array_equal(q["kbar"], kbars[h])
        # the key scale pins kbar: fl32((3 - kbar) / 448) changes with kbar's other tie neighbour
        kb = kbars[h][:nb]
        above = np.array([kexact[h][b] > float(kb[b]) for b in range(nb)])
        alt = np.where(above, np.nextafter(kb, np.float32(np.inf)), np.nextafter(kb, np.float32(-np.inf)))
        three = np.float32(3)
        assert np.array_equal(q["sK"], (three - kb) / np.float32(448))
        assert np.count_nonzero((three - kb) / np.float32(448) != (three - alt) / np.float32(448)) >= nb // 4
        assert np.array_equal(g["sK"][0, h], q["sK"]), h
        assert np.array_equal(g["Kq"][0, h], q["Kq"]), h
        assert np.array_equal(bf16_bits(out["mu"])[0, h].astype(np.int64), mus[h]), h
        for k in ("Qq", "sQ", "sV", "mu_scaled"):
            assert np.array_equal(g[k][0, h], q[k]), (h, k)
        assert np.array_equal(vq_rowmajor(g["Vq"])[0, h], q["Vq"]), h


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lam", [0.0, 2.0 ** -18])
def test_cluster_near_ties_beyond_binary64(d, lam):
    """The assignment where the best centroids' distances agree in every bit binary64 keeps:
    two-way near ties (decided by the token's own exact pair of distances) and three-way
    ones (the batched exact re-rank), ragged last work-group; with lam > 0 the size-penalised
    variant, sizes equal within a triple. Labels against the exact argmin and, with perm and
    centroids, against the oracle."""
    B, H, N, T = 1, 2, 1152, 8
    K = 3 * T
    rng = np.random.default_rng(100 + d)
    hs = [ws.near_tie_tokens(rng, N, d, T) for _ in range(H)]
    V = np.stack([x[0] for x in hs])[None]
    C0 = np.stack([x[1] for x in hs])[None]
    C = to_dev(C0)
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty_like(lab)
    cnt0 = np.broadcast_to(np.repeat(10 + np.arange(T), 3).astype(np.int32), (B, H, K)).copy()
    if lam == 0.0:
        vc.vc_cluster(to_dev_bf16(V), K, 1, False, C, lab, perm)
    else:
        cnt = to_dev(cnt0)
        vc.vc_cluster_balanced(to_dev_bf16(V), K, 1, False, lam, cnt, C, lab, perm)
    torch.cuda.synchronize()
    lg, pg, Cg = lab.cpu().numpy(), perm.cpu().numpy(), C.cpu().numpy()
    for h in range(H):
        Vf = synth.bf16_to_f32(V[0, h]).astype(np.float64)
        near = hs[h][2]
        for t in range(0, N, 7):  # exact argmin over the token's triple (the rest are far)
            cand = [3 * near[t] + m for m in range(3)]
            ex = [ws.exact_sqdist(Vf[t], C0[0, h, k]) for k in cand]
            assert lg[0, h, t] == cand[int(np.argmin(ex))], (h, t)
        if lam == 0.0:
            l_or, p_or, c_or = oracle.kmeans(V[0, h], K, 1, cold=False, C=C0[0, h])
        else:
            l_or, p_or, c_or, n_or = oracle.kmeans_balanced(V[0, h], K, 1, False, lam, cnt0[0, h], C0[0, h])
            assert np.array_equal(cnt.cpu().numpy()[0, h], n_or), h
        assert np.array_equal(lg[0, h], l_or), (h, np.count_nonzero(lg[0, h] != l_or))
        assert np.array_equal(pg[0, h], p_or), h
        assert np.array_equal(Cg[0, h], c_or), h


@pytest.mark.parametrize("d", [64, 128])
def test_means_on_subnormal_grids(d):
    """Values m 2^-133 (bfloat16 subnormals and the smallest normals): the k-means centroid
    (one cluster of 384 tokens) on the binary32 subnormal grid and the quantiser's block
    means on the bfloat16 subnormal grid, against the oracle and the rational results (the
    residual codes are outside the quantiser's range here: 448/amax overflows)."""
    from fractions import Fraction as F
    B, H, N = 1, 2, 384
    rng = np.random.default_rng(110 + d)
    X = np.stack([ws.tiny_values(rng, N, d).astype(np.float32) for _ in range(H)])[None]
    V = synth.bf16_bits(X)
    C0 = np.zeros((B, H, 1, d), np.float32)
    C = to_dev(C0)
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty_like(lab)
    vc.vc_cluster(to_dev_bf16(V), 1, 1, False, C, lab, perm)
    Q = np.stack([synth.gen_head("wan", 111, 0, h, N, d)["Q"] for h in range(H)])[None]
    flags = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH
    out = gpu_quantize(Q, Q, V, None, flags)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    for h in range(H):
        exp = np.array([ws.f32_of_tiny(sum(F(float(x)) for x in X[0, h, :, c]) / N) for c in range(d)], np.float32)
        _, _, c_or = oracle.kmeans(V[0, h], 1, 1, cold=False, C=C0[0, h])
        assert np.array_equal(c_or[0], exp), h
        assert np.array_equal(Cg[0, h], c_or), h
        q = oracle.quantize(Q[0, h], Q[0, h], V[0, h], None, int(flags))
        assert np.array_equal(bf16_bits(out["mu"])[0, h], q["mu"]), h


@pytest.mark.parametrize("d", [64, 128])
def test_cluster_near_ties_at_the_distance_span_limit(d):
    """Near ties as above with tokens and centroids spanning exactly 50 - log2 d binary
    exponents (the limit up to which the squared distances are exact, include/vc.h): the
    checker reports that span, and labels, perm and centroids equal the oracle's and the
    exact argmin."""
    B, H, N, T = 1, 2, 1152, 8
    K = 3 * T
    span = 50 - int(np.log2(d))
    rng = np.random.default_rng(120 + d)
    hs = [ws.near_tie_tokens(rng, N, d, T, tiny_exp=11 - span) for _ in range(H)]
    V = np.stack([x[0] for x in hs])[None]
    C0 = np.stack([x[1] for x in hs])[None]
    sv = vc.vc_exponent_span(to_dev_bf16(V)).cpu().numpy()[0]
    sc = vc.vc_exponent_span(to_dev(C0), as_bf16=True).cpu().numpy()[0]
    for h in range(H):
        assert max(sv[h][0], sc[h][0]) - min(sv[h][1], sc[h][1]) == span, (h, sv[h], sc[h])
    C = to_dev(C0)
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty_like(lab)
    vc.vc_cluster(to_dev_bf16(V), K, 1, False, C, lab, perm)
    torch.cuda.synchronize()
    lg, pg, Cg = lab.cpu().numpy(), perm.cpu().numpy(), C.cpu().numpy()
    for h in range(H):
        Vf = synth.bf16_to_f32(V[0, h]).astype(np.float64)
        near = hs[h][2]
        for t in range(0, N, 7):
            cand = [3 * near[t] + m for m in range(3)]
            ex = [ws.exact_sqdist(Vf[t], C0[0, h, k]) for k in cand]
            assert lg[0, h, t] == cand[int(np.argmin(ex))], (h, t)
        l_or, p_or, c_or = oracle.kmeans(V[0, h], K, 1, cold=False, C=C0[0, h])
        assert np.array_equal(lg[0, h], l_or), (h, np.count_nonzero(lg[0, h] != l_or))
        assert np.array_equal(pg[0, h], p_or), h
        assert np.array_equal(Cg[0, h], c_or), h


@pytest.mark.parametrize("d", [64, 128])
def test_cluster_means_at_the_sum_span_limit(d):
    """Centroid means whose values span exactly 103 - 2 ceil(log2 N) binary exponents over
    the head (the limit up to which the member sums are exact, include/vc.h; 83 at N = 1024):
    the checker reports that span, and the centroids equal the oracle's and the exact means
    rounded once."""
    B, H, K, n = 1, 2, 4, 256
    N = K * n
    span = 103 - 2 * int(np.ceil(np.log2(N)))
    rng = np.random.default_rng(130 + d)
    # E = 6 (the identity channels' 64); lowest bit 8 - g of the offset pieces n 2^-g
    g = 8 - (6 - span)
    heads = [_clustered_head(rng, d, (n,) * K, lambda r, m, c: ws.mean_columns(r, m, c, "f32", g=g)[::2])
             for _ in range(H)]
    V = np.stack([synth.bf16_bits(h[0].astype(np.float32)) for h in heads])[None]
    sv = vc.vc_exponent_span(to_dev_bf16(V)).cpu().numpy()[0]
    for h in range(H):
        assert sv[h][0] - sv[h][1] == span, (h, sv[h])
    C0 = np.zeros((B, H, K, d), np.float32)
    for k in range(K):
        C0[..., k, k] = 64.0
    C = to_dev(C0)
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty_like(lab)
    vc.vc_cluster(to_dev_bf16(V), K, 1, False, C, lab, perm)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    for h in range(H):
        _, _, c_or = oracle.kmeans(V[0, h], K, 1, cold=False, C=C0[0, h])
        assert np.array_equal(Cg[0, h], c_or), (h, np.count_nonzero(Cg[0, h] != c_or))
        for k in range(K):
            assert np.array_equal(Cg[0, h, k, K:], heads[h][2][k]), (h, k)


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_means_at_the_sum_span_limits(d):
    """Block means with V spanning exactly 89 binary exponents (the limit for 128-term sums)
    and the key mean with K spanning exactly 83 (the limit for N = 1024 terms), both next to
    rounding ties: the checker reports those spans, the oracle's means equal the rational
    ones, and every quantiser output equals the oracle's."""
    B, H, N = 1, 2, 1024
    nb = N // 128
    rng = np.random.default_rng(140 + d)
    Qs, Ks, Vs, perms, mus, kbars = [], [], [], [], [], []
    for h in range(H):
        Vp = np.zeros((N, d))
        mu = np.zeros((nb, d), np.int64)
        for b in range(nb):  # E = 6 (pairs), lowest bit 7 - g of the offsets 128 2^-g: span g - 1
            X, _, r = ws.mean_columns(rng, 128, d, "bf16", g=90)
            Vp[128 * b:128 * (b + 1)] = X
            mu[b] = r
        perm = synth.rand_perm(N, 141, 0, h)
        V = np.zeros_like(Vp)
        V[perm] = Vp
        Kx, _, kb = ws.mean_columns(rng, N, d, "f32", small=True, g=92)  # E = 1, lowest bit 10 - g
        Qs.append(synth.gen_head("wan", 142, 0, h, N, d)["Q"])
        Ks.append(synth.bf16_bits(Kx.astype(np.float32)))
        Vs.append(synth.bf16_bits(V.astype(np.float32)))
        perms.append(perm)
        mus.append(mu)
        kbars.append(np.array(kb, np.float32))
    Q, K, V, P = (np.stack(x)[None] for x in (Qs, Ks, Vs, perms))
    sv = vc.vc_exponent_span(to_dev_bf16(V)).cpu().numpy()[0]
    sk = vc.vc_exponent_span(to_dev_bf16(K)).cpu().numpy()[0]
    for h in range(H):
        assert sv[h][0] - sv[h][1] == 103 - 2 * 7 and sk[h][0] - sk[h][1] == 103 - 2 * 10, (h, sv[h], sk[h])
    flags = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH
    out = gpu_quantize(Q, K, V, P, flags)
    g = {k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in out.items()}
    for h in range(H):
        q = oracle.quantize(Q[0, h], K[0, h], V[0, h], P[0, h], int(flags))
        assert np.array_equal(q["mu"].astype(np.int64), mus[h])
        assert np.array_equal(q["kbar"], kbars[h])
        assert np.array_equal(bf16_bits(out["mu"])[0, h].astype(np.int64), mus[h]), h
        for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu_scaled"):
            assert np.array_equal(g[k][0, h], q[k]), (h, k)
        assert np.array_equal(vq_rowmajor(g["Vq"])[0, h], q["Vq"]), h
