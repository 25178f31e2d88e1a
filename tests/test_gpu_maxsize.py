"""Parity at the largest shape the ABI accepts: B=2, H=60, N=131,072, d=128, so that
B*H*N*d = 2,013,265,920 sits just under the 2^31 element limit.

Every head holds different data. The first and the last (b,h) are heads of the video
workload's generator (clustered values with outlier tokens, biased keys; seeds of their
own), the heads between are seeded device random tensors. The two generated heads are
checked against the oracle computed from their own inputs: k-means labels, permutation
and centroids and every quantiser output bit-exact, and attention on sampled rows
(including token N-1 and the last key block) within the path's 2e-3 tolerance. Offsets
that overflow 32 bits, or a head index mapped onto the wrong data, fail here first.

A third checked head, (0, 1), holds zero-mean Gaussian Q, K, V (the ExpCast-only
workload's recipe) over all 131k keys, where the output is small relative to the values.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402

vc = pytest.importorskip("bit_attention_video_online_amd")
from tests.gpu_util import bf16_bits, emul, rel_l2, vq_rowmajor  # noqa: E402

B, H, N, D = 2, 60, 131072, 128
KC = 512
ITERS = 2
BETA = oracle.BETA_E4M3
GAUSS = (0, 1)
CHECKED = ((0, 0), GAUSS, (B - 1, H - 1))


def _head_to_dev(t, bits, b, h):
    t[b, h].copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16))


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert B * H * N * D < 2 ** 31
    print("\n[maxsize] B=%d H=%d N=%d d=%d: generating" % (B, H, N, D), flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    Q = torch.randn((B, H, N, D), generator=g, device="cuda").to(torch.bfloat16)
    K = (torch.randn((B, H, N, D), generator=g, device="cuda") + 2.0).to(torch.bfloat16)
    V = (torch.randn((B, H, N, D), generator=g, device="cuda") * 3.0).to(torch.bfloat16)
    # the checked heads: the video workload's generator, and zero-mean Gaussian values
    for (b, h) in CHECKED:
        w = synth.gen_head("expcast", 46, b, h, N, D) if (b, h) == GAUSS else synth.gen_head("sweep", 45, b, h, N, D)
        for t, k in ((Q, "Q"), (K, "K"), (V, "V")):
            _head_to_dev(t, w[k], b, h)
    C = torch.zeros((B, H, KC, D), dtype=torch.float32, device="cuda")
    lab = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    print("[maxsize] k-means", flush=True)
    vc.vc_cluster(V, KC, ITERS, True, C, lab, perm)
    q = vc.quantize_outputs(B, H, N, D)
    print("[maxsize] quantise", flush=True)
    vc.vc_quantize(Q, K, V, perm, vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH, q)
    O = torch.empty((B, H, N, D), dtype=torch.bfloat16, device="cuda")
    print("[maxsize] attention", flush=True)
    vc.vc_attention(q, O, beta=BETA, flags=vc.VC_F_EXPCAST)
    torch.cuda.synchronize()
    print("[maxsize] GPU path done", flush=True)
    res = {}
    for (b, h) in CHECKED:
        res[(b, h)] = dict(
            Q=bf16_bits(Q[b, h]), K=bf16_bits(K[b, h]), V=bf16_bits(V[b, h]),
            lab=lab[b, h].cpu().numpy(), perm=perm[b, h].cpu().numpy(), C=C[b, h].cpu().numpy(),
            q={k: (bf16_bits(v[b, h]) if v.dtype == torch.bfloat16 else v[b, h].cpu().numpy()) for k, v in q.items()},
            O=bf16_bits(O[b, h]))
    del Q, K, V, C, lab, perm, q, O
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("bh", CHECKED)
def test_maxsize_head_matches_oracle(big, bh):
    r = big[bh]
    print("[maxsize] oracle for head %s" % (bh,), flush=True)
    lab, perm, C = oracle.kmeans(r["V"], KC, ITERS, cold=True)
    assert np.array_equal(r["lab"], lab)
    assert np.array_equal(r["perm"], perm)
    assert np.array_equal(r["C"], C)
    o = oracle.quantize(r["Q"], r["K"], r["V"], perm, oracle.FLAG_KSMOOTH | oracle.FLAG_VSMOOTH)
    g = r["q"]
    for k in ("Qq", "sQ", "Kq", "sK", "sV", "mu", "mu_scaled"):
        assert np.array_equal(g[k], o[k]), k
    assert np.array_equal(vq_rowmajor(g["Vq"][None, None])[0, 0], o["Vq"])
    rng = np.random.default_rng(91)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)])).astype(np.int32)
    O_em = emul(o, rows, beta=BETA, mode=oracle.MODE_EXPCAST)
    err = rel_l2(synth.bf16_to_f32(r["O"][rows]).astype(np.float64), O_em)
    print("[maxsize] head %s: rel-L2 vs emulation %.2e" % (bh, err), flush=True)
    assert err <= 2e-3
