"""Parity at the full Wan2.2-shaped size (B=1, H=40, N=70,400, d=128, 550 clusters),
in the launch configuration that bench.py times.

The GPU runs the whole batch; the oracle recomputes two sampled heads completely
(k-means warm start and both iterations, quantiser) and 64 query rows per sampled head
for attention (rows are independent given K and V). Properties that hold at any size
(pi is a stable sort of the labels) are checked on every head. In-kernel ExpCast bytes of the
first and the last key block are bit-exact on sampled rows. The error of the VC path
against binary64 exact attention is compared with the plain FP8 path.
"""
import time

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402

vc = pytest.importorskip("bit_attention_video_online_amd")
from tests.gpu_util import bf16_bits, emul, mu_pack_expected, rel_l2, to_dev_bf16, vq_rowmajor  # noqa: E402

HEADS = (0, 23)
KC = 550
BETA = oracle.BETA_E4M3


@pytest.fixture(scope="module")
def run():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    t0 = time.time()
    w = synth.gen("wan")
    print("\n[wan] inputs generated in %.1fs" % (time.time() - t0), flush=True)
    B, H, N, d = w["Q"].shape
    Q, K, V, Vp = (to_dev_bf16(w[k]) for k in ("Q", "K", "V", "V_prev"))
    Cw = torch.zeros((B, H, KC, d), dtype=torch.float32, device="cuda")
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    vc.vc_cluster(Vp, KC, 4, True, Cw, lab, perm)
    C = Cw.clone()
    vc.vc_cluster(V, KC, 2, False, C, lab, perm)
    q = vc.quantize_outputs(B, H, N, d)
    vc.vc_quantize(Q, K, V, perm, vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH, q)
    O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    vc.vc_attention(q, O, beta=BETA, flags=vc.VC_F_EXPCAST)
    # comparison paths: V-Smooth with exp-then-cast, plain FP8 (no V-Smooth, exp then cast), ExpCast only
    Ovs = torch.empty_like(O)
    vc.vc_attention(q, Ovs, beta=BETA, flags=0)
    qp = vc.quantize_outputs(B, H, N, d)
    vc.vc_quantize(Q, K, V, None, vc.VC_F_KSMOOTH, qp)
    Op = torch.empty_like(O)
    vc.vc_attention(qp, Op, beta=BETA, flags=0, restore_mean=False)
    Oe = torch.empty_like(O)
    vc.vc_attention(qp, Oe, beta=BETA, flags=vc.VC_F_EXPCAST, restore_mean=False)
    dumps = {}
    codes = torch.empty((B, H, N, 128), dtype=torch.uint8, device="cuda")
    for blk in (0, N // 128 - 1):
        Od = torch.empty_like(O)
        vc.vc_attention_dump(q, Od, blk, codes, beta=BETA, flags=vc.VC_F_EXPCAST)
        torch.cuda.synchronize()
        dumps[blk] = (codes[:, list(HEADS)].cpu().numpy(), bool(torch.equal(Od, O)))
        del Od
    del codes
    O5 = torch.empty_like(O)  # the VC path with E5M2 ExpCast bytes
    vc.vc_attention(q, O5, beta=oracle.BETA_E5M2, flags=vc.VC_F_EXPCAST | vc.VC_F_E5M2)
    # the same launch repeated on the same inputs: any race between the waves of a
    # work-group (tile stages overwritten while still being read) shows up as a difference
    repeat_identical = []
    for _ in range(4):
        Or = torch.empty_like(O)
        vc.vc_attention(q, Or, beta=BETA, flags=vc.VC_F_EXPCAST)
        repeat_identical.append(bool(torch.equal(Or, O)))
        del Or
    # one repeat of each other attention variant (exp-then-cast, plain FP8, E5M2 bytes)
    for qq, ref, beta, flags, rm in ((q, Ovs, BETA, 0, True), (qp, Op, BETA, 0, False),
                                     (q, O5, oracle.BETA_E5M2, vc.VC_F_EXPCAST | vc.VC_F_E5M2, True)):
        Or = torch.empty_like(O)
        vc.vc_attention(qq, Or, beta=beta, flags=flags, restore_mean=rm)
        repeat_identical.append(bool(torch.equal(Or, ref)))
        del Or
    # k-means (warm, from the same start) and the quantiser repeated as well
    C2 = Cw.clone()
    lab2, perm2 = torch.empty_like(lab), torch.empty_like(perm)
    vc.vc_cluster(V, KC, 2, False, C2, lab2, perm2)
    repeat_identical.append(bool(torch.equal(C2, C) and torch.equal(lab2, lab) and torch.equal(perm2, perm)))
    q2 = vc.quantize_outputs(B, H, N, d)
    vc.vc_quantize(Q, K, V, perm, vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH, q2)
    repeat_identical.append(all(bool(torch.equal(q2[k], q[k])) for k in q))
    del C2, lab2, perm2, q2
    torch.cuda.synchronize()
    print("[wan] GPU path done in %.1fs" % (time.time() - t0), flush=True)
    res = dict(w=w, Cw=Cw.cpu().numpy(), C=C.cpu().numpy(), lab=lab.cpu().numpy(), perm=perm.cpu().numpy(),
               q={k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in q.items()},
               O=bf16_bits(O), Ovs=bf16_bits(Ovs), Op=bf16_bits(Op), Oe=bf16_bits(Oe), O5=bf16_bits(O5),
               repeat_identical=repeat_identical, dumps=dumps)
    del Q, K, V, Vp, q, qp, O, Op, Ovs, Oe, O5
    torch.cuda.empty_cache()
    return res


def test_wan_attention_repeatable(run):
    """Four more launches of the VC attention on the same inputs give the same bytes, as do one
    more launch of each other attention variant (exp-then-cast, plain FP8, E5M2 bytes), a second
    warm k-means from the same centroids and a second quantiser call: every
    accumulation order is fixed, so any difference is a race (for attention, a tile stage
    copied over while another wave of the work-group still reads it)."""
    assert all(run["repeat_identical"]), run["repeat_identical"]


def test_wan_perm_is_stable_sort_all_heads(run):
    lab, perm = run["lab"], run["perm"]
    for h in range(lab.shape[1]):
        assert np.array_equal(perm[0, h], np.argsort(lab[0, h], kind="stable")), h
        assert lab[0, h].min() >= 0 and lab[0, h].max() < KC


@pytest.fixture(scope="module")
def oracle_heads(run):
    w = run["w"]
    out = {}
    for h in HEADS:
        t0 = time.time()
        _, _, Cw = oracle.kmeans(w["V_prev"][0, h], KC, 4, cold=True)
        lab, perm, C = oracle.kmeans(w["V"][0, h], KC, 2, cold=False, C=Cw)
        q = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
        out[h] = dict(Cw=Cw, lab=lab, perm=perm, C=C, q=q)
        print("[wan] oracle head %d in %.1fs" % (h, time.time() - t0), flush=True)
    return out


def test_wan_kmeans_bitexact_sampled_heads(run, oracle_heads):
    for h in HEADS:
        o = oracle_heads[h]
        assert np.array_equal(run["Cw"][0, h], o["Cw"]), h
        assert np.array_equal(run["lab"][0, h], o["lab"]), h
        assert np.array_equal(run["perm"][0, h], o["perm"]), h
        assert np.array_equal(run["C"][0, h], o["C"]), h


def test_wan_cluster_cost_sampled_heads(run, oracle_heads):
    """The drift statistic at full size: k-means objective of V under the warm-started
    clustering, all heads on the GPU, two heads against the oracle (relative 1e-11)."""
    w = run["w"]
    B, H, N, d = w["V"].shape
    cost = torch.empty((B, H), dtype=torch.float64, device="cuda")
    vc.vc_cluster_cost(to_dev_bf16(w["V"]), torch.from_numpy(run["C"]).cuda(), torch.from_numpy(run["lab"]).cuda(),
                       cost)
    got = cost.cpu().numpy()
    for h in HEADS:
        want = oracle.kmeans_cost(w["V"][0, h], oracle_heads[h]["C"], oracle_heads[h]["lab"])
        assert abs(got[0, h] - want) <= 1e-11 * want, (h, got[0, h], want)
    assert np.all(got > 0)


def test_wan_balanced_kmeans_sampled_heads(run, oracle_heads):
    """Size-penalised k-means at full size from the warm state (sizes of the warm labels),
    lambda = 0.01 J / (N/K): all heads on the GPU, two heads bit-exact against the oracle."""
    w = run["w"]
    B, H, N, d = w["V"].shape
    # inputs of the sampled heads come from the oracle (its warm state and the sizes of its
    # warm-started labels); the other heads start from the GPU warm state with zero sizes
    Cw = run["Cw"].copy()
    cnt0 = np.zeros((B, H, KC), np.int32)
    for h in HEADS:
        Cw[0, h] = oracle_heads[h]["Cw"]
        cnt0[0, h] = np.bincount(oracle_heads[h]["lab"], minlength=KC)
    lam = float(np.float32(0.01 * 141.87 * KC / N))
    C = torch.from_numpy(Cw).cuda()
    cnt = torch.from_numpy(cnt0).cuda()
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    vc.vc_cluster_balanced(to_dev_bf16(w["V"]), KC, 2, False, lam, cnt, C, lab, perm)
    torch.cuda.synchronize()
    lab, perm, C, cnt = (x.cpu().numpy() for x in (lab, perm, C, cnt))
    for h in HEADS:
        l_or, p_or, c_or, n_or = oracle.kmeans_balanced(w["V"][0, h], KC, 2, False, lam, cnt0[0, h], Cw[0, h])
        assert np.array_equal(lab[0, h], l_or), (h, np.count_nonzero(lab[0, h] != l_or))
        assert np.array_equal(perm[0, h], p_or), h
        assert np.array_equal(C[0, h], c_or), h
        assert np.array_equal(cnt[0, h], n_or), h
    for h in range(H):
        assert np.array_equal(cnt[0, h], np.bincount(lab[0, h], minlength=KC)), h


def test_wan_incremental_update_sampled_heads(run, oracle_heads):
    """One cross-step incremental step at full size (decay 1/2, re-assignment) from the warm
    state, with masses from the warm labels: all heads on the GPU, two heads bit-exact."""
    w = run["w"]
    B, H, N, d = w["V"].shape
    C = run["Cw"].copy()
    M = np.zeros((B, H, KC), np.float32)
    for h in HEADS:
        C[0, h] = oracle_heads[h]["Cw"]
        M[0, h] = np.bincount(oracle_heads[h]["lab"], minlength=KC)
    Cd, Md = torch.from_numpy(C).cuda(), torch.from_numpy(M).cuda()
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    vc.vc_cluster_incremental(to_dev_bf16(w["V"]), 0.5, True, Cd, Md, lab, perm)
    torch.cuda.synchronize()
    lab, perm, Cd, Md = (x.cpu().numpy() for x in (lab, perm, Cd, Md))
    for h in HEADS:
        l_or, p_or, c_or, m_or = oracle.kmeans_incremental(w["V"][0, h], C[0, h], M[0, h], 0.5, True)
        assert np.array_equal(lab[0, h], l_or), (h, np.count_nonzero(lab[0, h] != l_or))
        assert np.array_equal(perm[0, h], p_or), h
        assert np.array_equal(Cd[0, h], c_or), h
        assert np.array_equal(Md[0, h], m_or), h


def test_wan_quantize_bitexact_sampled_heads(run, oracle_heads):
    g = run["q"]
    for h in HEADS:
        o = oracle_heads[h]["q"]
        assert np.array_equal(g["Qq"][0, h], o["Qq"])
        assert np.array_equal(g["sQ"][0, h], o["sQ"])
        assert np.array_equal(g["Kq"][0, h], o["Kq"])
        assert np.array_equal(g["sK"][0, h], o["sK"])
        assert np.array_equal(vq_rowmajor(g["Vq"])[0, h], o["Vq"])
        assert np.array_equal(g["sV"][0, h], o["sV"])
        assert np.array_equal(g["mu"][0, h], o["mu"])
        assert np.array_equal(g["mu_scaled"][0, h], o["mu_scaled"])
        assert np.array_equal(g["mu_pack"][0, h], mu_pack_expected(o["mu_scaled"]))


@pytest.fixture(scope="module")
def sampled_errors(run, oracle_heads):
    """Output of every path on 64 seeded rows of the sampled heads: against the emulation, and
    against binary64 exact attention (rMSE = ||O - O_exact|| / ||O_exact||)."""
    w = run["w"]
    N = w["Q"].shape[2]
    rng = np.random.default_rng(77)
    errs, errs5, errs_x = [], [], []
    e = {k: [] for k in ("vc", "vsmooth", "plain", "expcast", "vc_e5m2")}
    for h in HEADS:
        rows = np.sort(rng.choice(N, 64, replace=False)).astype(np.int32)
        got = lambda key: synth.bf16_to_f32(run[key][0, h][rows]).astype(np.float64)
        errs.append(rel_l2(got("O"), emul(oracle_heads[h]["q"], rows, beta=BETA, mode=oracle.MODE_EXPCAST)))
        errs5.append(rel_l2(got("O5"), emul(oracle_heads[h]["q"], rows, beta=oracle.BETA_E5M2,
                                              mode=oracle.MODE_EXPCAST_E5M2)))
        errs_x.append(rel_l2(got("O"), oracle.attention_emul(oracle_heads[h]["q"], rows, beta=BETA,
                                                              mode=oracle.MODE_EXPCAST)))
        O_ex = oracle.attention_exact(w["Q"][0, h], w["K"][0, h], w["V"][0, h], rows)
        for k, key in (("vc", "O"), ("vsmooth", "Ovs"), ("plain", "Op"), ("expcast", "Oe"), ("vc_e5m2", "O5")):
            e[k].append(rel_l2(got(key), O_ex))
    m = {k: float(np.mean(v)) for k, v in e.items()}
    print("[wan] rel-L2 vs emulation %s (E5M2 %s; exactly rounded scores, unrounded output %s); rMSE vs exact %s"
          % (errs, errs5, errs_x, m), flush=True)
    return dict(errs=errs, errs5=errs5, rmse=m)


def test_wan_attention_sampled_rows(sampled_errors):
    """Output within rel-L2 2e-3 of the emulation for E4M3 and E5M2 bytes; V-Smooth lowers the
    error of each probability quantiser it is added to."""
    s = sampled_errors
    assert max(s["errs"]) <= 2e-3
    assert max(s["errs5"]) <= 2e-3
    assert s["rmse"]["vsmooth"] < s["rmse"]["plain"]
    assert s["rmse"]["vc"] < s["rmse"]["expcast"]


@pytest.mark.xfail(reason="on this generator (64 value centres of norm 4 under per-element noise of std 1, so a "
                          "128-token block shares little of its value) the probability term dominates the error and "
                          "ExpCast's code costs about as much as V-Smooth saves: VC 0.852 %, plain FP8 0.836 % "
                          "measured (64 rows x 2 heads); with tight value clusters VC is below plain FP8 "
                          "(test_gpu_wan_tight)", strict=False)
def test_wan_vc_error_below_plain_fp8(sampled_errors):
    """The VC path (V-Smooth + ExpCast) against plain FP8 (exp then cast, no V-Smooth), error
    against binary64 exact attention on the sampled rows."""
    m = sampled_errors["rmse"]
    assert m["vc"] < m["plain"], (m["vc"], m["plain"])


def test_wan_inkernel_bytes_first_and_last_block(run, oracle_heads):
    """ExpCast bytes inside the attention loop at full size, key blocks 0 and 549 (after the
    running maximum has evolved over all of them), 128 sampled rows of two heads: bit-exact."""
    N = run["w"]["Q"].shape[2]
    rng = np.random.default_rng(81)
    for blk, (codes, same_output) in run["dumps"].items():
        assert same_output
        for i, h in enumerate(HEADS):
            rows = np.sort(rng.choice(N, 128, replace=False)).astype(np.int32)
            _, c_or = emul(oracle_heads[h]["q"], rows, beta=BETA, mode=oracle.MODE_EXPCAST, dump_block=blk)
            got = codes[0, i][rows]
            assert np.array_equal(got, c_or), (blk, h, np.count_nonzero(got != c_or))


def test_wan_every_head_bitexact_and_rows(run):
    """Every one of the 40 heads against the oracle: warm-start and warm k-means (centroids,
    labels, pi), every quantiser output bit-exact, and the VC output on 32 seeded rows per
    head within 2e-3 of the emulation (rows are independent given K and V)."""
    w = run["w"]
    g = run["q"]
    B, H, N, d = w["Q"].shape
    rng = np.random.default_rng(80)
    worst = 0.0
    t0 = time.time()
    for h in range(H):
        _, _, Cw = oracle.kmeans(w["V_prev"][0, h], KC, 4, cold=True)
        lab, perm, C = oracle.kmeans(w["V"][0, h], KC, 2, cold=False, C=Cw)
        assert np.array_equal(run["Cw"][0, h], Cw), h
        assert np.array_equal(run["lab"][0, h], lab), h
        assert np.array_equal(run["perm"][0, h], perm), h
        assert np.array_equal(run["C"][0, h], C), h
        o = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
        for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu", "mu_scaled"):
            assert np.array_equal(g[k][0, h], o[k]), (h, k)
        assert np.array_equal(vq_rowmajor(g["Vq"])[0, h], o["Vq"]), h
        rows = np.sort(rng.choice(N, 32, replace=False)).astype(np.int32)
        O_em = emul(o, rows, beta=BETA, mode=oracle.MODE_EXPCAST)
        err = rel_l2(synth.bf16_to_f32(run["O"][0, h][rows]).astype(np.float64), O_em)
        worst = max(worst, err)
        assert err <= 2e-3, (h, err)
        if h % 8 == 7:
            print("[wan] heads 0-%d match (%.0fs, worst rel-L2 %.2e)" % (h, time.time() - t0, worst), flush=True)


def test_wan_rope_hadamard_sampled_heads(run, oracle_heads):
    """RoPE on the video grid (22 x 40 x 80) and the Q/K Hadamard rotation inside the
    quantiser at full size: quantiser outputs of two heads bit-exact, attention on sampled
    rows within 2e-3 of the emulation; error against exact attention on the RoPE'd inputs
    printed for the path with and without the rotation."""
    w = run["w"]
    B, H, N, d = w["Q"].shape
    tabs = synth.rope_tables(N, d, synth.WAN_GRID)
    rc, rs = (torch.from_numpy(t).cuda() for t in tabs)
    Q, K, V = (to_dev_bf16(w[k]) for k in ("Q", "K", "V"))
    perm = torch.from_numpy(run["perm"]).cuda()
    res = {}
    for had in (False, True):
        flags = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH | (vc.VC_F_HADAMARD if had else 0)
        q = vc.quantize_outputs(B, H, N, d)
        vc.vc_quantize(Q, K, V, perm, flags, q, rope_cos=rc, rope_sin=rs)
        O = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        vc.vc_attention(q, O, beta=BETA, flags=vc.VC_F_EXPCAST)
        torch.cuda.synchronize()
        res[had] = ({k: (bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in q.items()},
                    bf16_bits(O))
        del q, O
    del Q, K, V
    torch.cuda.empty_cache()
    rng = np.random.default_rng(78)
    err_ex = {False: [], True: []}
    for h in HEADS:
        rows = np.sort(rng.choice(N, 64, replace=False)).astype(np.int32)
        O_ex = oracle.attention_exact(oracle.rope(w["Q"][0, h], *tabs), oracle.rope(w["K"][0, h], *tabs),
                                      w["V"][0, h], rows)
        for had in (False, True):
            g, O = res[had]
            o = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], oracle_heads[h]["perm"],
                                oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH | (oracle.FLAG_HADAMARD if had else 0),
                                rope_cos=tabs[0], rope_sin=tabs[1])
            for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu_scaled"):
                assert np.array_equal(g[k][0, h], o[k]), (had, h, k)
            assert np.array_equal(vq_rowmajor(g["Vq"])[0, h], o["Vq"])
            got = synth.bf16_to_f32(O[0, h][rows]).astype(np.float64)
            O_em = emul(o, rows, beta=BETA, mode=oracle.MODE_EXPCAST)
            assert rel_l2(got, O_em) <= 2e-3, (had, h)
            err_ex[had].append(rel_l2(got, O_ex))
    print("[wan rope] rMSE vs exact on the RoPE'd inputs: without rotation %.4f, with Hadamard %.4f"
          % (np.mean(err_ex[False]), np.mean(err_ex[True])), flush=True)


def test_wan_mxfp4_sampled_rows(run, oracle_heads):
    """The 4-bit (MXFP4) value residual at full size with the warm-started permutation:
    exp-then-cast + V-Smooth (the pages' 4-bit configuration) and ExpCast + V-Smooth, sampled
    rows of two heads within 2e-3 of the emulation; group scales and codes of the sampled
    heads bit-exact; error against exact attention printed beside the 8-bit path."""
    from tests.gpu_util import mx_unpack
    w = run["w"]
    B, H, N, d = w["Q"].shape
    Q, K, V = (to_dev_bf16(w[k]) for k in ("Q", "K", "V"))
    perm = torch.from_numpy(run["perm"]).cuda()
    flags = vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH | vc.VC_F_MXFP4
    q = vc.quantize_outputs(B, H, N, d)
    vc.vc_quantize(Q, K, V, perm, flags, q)
    O = {}
    for name, af in (("exp", vc.VC_F_MXFP4), ("vc", vc.VC_F_EXPCAST | vc.VC_F_MXFP4)):
        O[name] = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        vc.vc_attention(q, O[name], beta=BETA, flags=af)
    torch.cuda.synchronize()
    codes, scales = mx_unpack(q["Vq"].cpu().numpy())
    O = {k: bf16_bits(v) for k, v in O.items()}
    del Q, K, V, q
    torch.cuda.empty_cache()
    rng = np.random.default_rng(79)
    err_ex = {"exp": [], "vc": []}
    for h in HEADS:
        o = oracle.quantize(w["Q"][0, h], w["K"][0, h], w["V"][0, h], oracle_heads[h]["perm"], int(flags))
        assert np.array_equal(codes[0, h], o["Vq"]) and np.array_equal(scales[0, h], o["Vs"]), h
        rows = np.sort(rng.choice(N, 64, replace=False)).astype(np.int32)
        O_ex = oracle.attention_exact(w["Q"][0, h], w["K"][0, h], w["V"][0, h], rows)
        for name, mode in (("exp", oracle.MODE_EXP_THEN_CAST), ("vc", oracle.MODE_EXPCAST)):
            got = synth.bf16_to_f32(O[name][0, h][rows]).astype(np.float64)
            assert rel_l2(got, emul(o, rows, beta=BETA, mode=mode)) <= 2e-3, (name, h)
            err_ex[name].append(rel_l2(got, O_ex))
    print("[wan mxfp4] rMSE vs exact: exp-then-cast + V-Smooth %.4f, ExpCast + V-Smooth %.4f"
          % (np.mean(err_ex["exp"]), np.mean(err_ex["vc"])), flush=True)
