"""Inputs on which the quantiser is exact, with every expected code, scale and mean known.

Q blocks are E4M3 values times a power of two with one element at 448 * 2^k (so the
block scale is 2^k). The smoothed, permuted keys K~' come in (x, -x) row pairs inside
every 128-row block (zero column mean) with block maximum 28 = 448/16; K = K~ + an
integer per-channel bias. The permuted values are V' = mu_j + R with R in (r, -r) row
pairs inside every block (zero block mean), per-channel maximum |R| = 14 = 448/32 and
mu_j a multiple of 1/8. Every value is exactly a bfloat16.
"""
import numpy as np

import synth

EVEN_E4M3 = np.array([2, 4, 6, 8, 10, 12, 14, 16, 20, 24, 28, 32, 40, 48, 56, 64, 80, 96, 112, 128,
                      160, 192, 224, 256, 320, 384, 448], np.float64)


def _e4m3_code_of(v):
    """Code of an exactly representable non-negative E4M3 value (test helper, small table)."""
    import oracle
    grid = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    idx = np.searchsorted(grid, v)
    assert np.all(grid[idx] == v)
    return idx.astype(np.uint8)


def representable_head(N=512, d=32, seed=0, permute=True, ksmooth_bias=True, vsmooth=True):
    rng = np.random.default_rng(seed)
    nb = N // 128
    perm = rng.permutation(N).astype(np.int32) if permute else np.arange(N, dtype=np.int32)
    # ---- Q
    grid = None
    import oracle
    grid = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    qcodes = rng.integers(1, 127, (N, d)).astype(np.uint8)
    qsign = rng.integers(0, 2, (N, d)).astype(np.uint8)
    kq = rng.integers(-3, 1, nb)
    for b in range(nb):
        r, c = rng.integers(0, 128), rng.integers(0, d)
        qcodes[b * 128 + r, c] = 126
    Qval = np.where(qsign == 1, -1.0, 1.0) * grid[qcodes]
    Qval = Qval * np.repeat(np.exp2(kq), 128)[:, None]
    exp_Qq = qcodes | (qsign << 7)
    # ---- K~' (permuted, smoothed)
    Kp = np.empty((N, d))
    for b in range(nb):
        x = rng.choice(EVEN_E4M3, (64, d)) * np.where(rng.integers(0, 2, (64, d)) == 1, -1.0, 1.0)
        x[rng.integers(0, 64), rng.integers(0, d)] = 448.0
        blk = np.concatenate([x, -x], 0)
        blk = blk[rng.permutation(128)]
        Kp[b * 128:(b + 1) * 128] = blk
    exp_Kq = _e4m3_code_of(np.abs(Kp)) | ((Kp < 0).astype(np.uint8) << 7)
    Kt_perm = Kp / 16.0
    Kt = np.empty_like(Kt_perm)
    Kt[perm] = Kt_perm
    bias = rng.integers(-3, 4, d).astype(np.float64) if ksmooth_bias else np.zeros(d)
    K = Kt + bias[None, :]
    # ---- V' = mu + R (permuted)
    R = np.empty((N, d))
    for b in range(nb):
        x = rng.choice(EVEN_E4M3[:20], (64, d)) * np.where(rng.integers(0, 2, (64, d)) == 1, -1.0, 1.0)
        blk = np.concatenate([x, -x], 0)
        R[b * 128:(b + 1) * 128] = blk[rng.permutation(128)]
    for c in range(d):   # per-channel maximum 448 somewhere (keeping the pair structure)
        b = rng.integers(0, nb)
        rows = np.nonzero(R[b * 128:(b + 1) * 128, c] == R[b * 128:(b + 1) * 128, c].max())[0]
        i = b * 128 + rows[0]
        partner = b * 128 + np.nonzero(R[b * 128:(b + 1) * 128, c] == -R[i, c])[0][0]
        R[i, c], R[partner, c] = 448.0, -448.0
    exp_Vq = _e4m3_code_of(np.abs(R)) | ((R < 0).astype(np.uint8) << 7)
    Rv = R / 32.0
    mu = (rng.integers(-14, 15, (nb, d)) / 8.0) if vsmooth else np.zeros((nb, d))
    Vp = Rv + np.repeat(mu, 128, 0)
    V = np.empty_like(Vp)
    V[perm] = Vp
    for arr in (Qval, K, V):
        assert np.array_equal(synth.bf16_to_f32(synth.bf16_bits(arr.astype(np.float32))), arr.astype(np.float32))
    return dict(
        Q=synth.bf16_bits(Qval.astype(np.float32)), K=synth.bf16_bits(K.astype(np.float32)),
        V=synth.bf16_bits(V.astype(np.float32)), perm=perm,
        exp=dict(Qq=exp_Qq, sQ_raw=np.exp2(kq).astype(np.float32), Kq=exp_Kq,
                 sK=np.full(nb, 1.0 / 16, np.float32), Vq=exp_Vq, sV=np.full(d, 1.0 / 32, np.float32),
                 mu=mu.astype(np.float32), kbar=bias.astype(np.float32)),
    )
