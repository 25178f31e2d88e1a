"""Seeded synthetic inputs shaped like the video-DiT attention workloads.

This module only draws random tensors; it contains none of the method's arithmetic,
so both the HIP path's tests and the CPU oracle can consume its output.

Every tensor is generated per (batch, head) from ``numpy.random.default_rng([seed,
tag, b, h])`` (PCG64), drawn in float32 and rounded to bfloat16 (round to nearest
even). Arrays are returned as raw bf16 bit patterns (``uint16``) in ``[B, H, N, d]``
layout, so any head can be regenerated on its own.

Workloads (stand-ins for the Wan2.2 attention tensors that the pages measure on,
which are not available):

* ``tiny``   -- B=1, H=1, N=1024, d=128: Q ~ N(0,1); K = N(0,1) + per-channel bias
  b ~ N(0, 3^2); V = mixture of 4 centres (norm 4) + N(0,1) noise, 2 % of tokens
  (20) multiplied by 20 on 8 channels.
* ``expcast`` -- B=1, H=8, N=8192, d=128: Q, K, V ~ N(0,1).
* ``wan``    -- B=1, H=40, N=70400, d=128: K as ``tiny``; V per head = 64 centres
  (norm 4, noise std 1) with 1 % outlier tokens (704) scaled by U[10,30] on 8 spike
  channels redrawn per head. ``V_prev`` is the previous denoising step's value
  tensor; ``V = bf16(V_prev + xi * |V_prev|)`` with xi ~ N(0, 0.05^2).
* ``sweep``  -- the ``wan`` generator at other (H, N, d).
* ``wan_tight`` -- B=1, H=2, N=70400, d=128: the ``wan`` recipe with tight value clusters
  (centre norm sqrt(d), i.e. about one per element, noise std 0.25), a model of highly
  redundant neighbouring video tokens; Q, K, outliers and drift as ``wan``.
"""
from __future__ import annotations

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_XI, TAG_PERM, TAG_MISC = 11, 12, 13, 14, 15, 16


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tag: int, b: int, h: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tag, b, h, step])


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def head_q(seed, b, h, N, d):
    return bf16_bits(_normal(_rng(seed, TAG_Q, b, h), (N, d)))


def head_k_biased(seed, b, h, N, d):
    rng = _rng(seed, TAG_K, b, h)
    bias = (3.0 * _normal(rng, (d,))).astype(np.float32)
    return bf16_bits(_normal(rng, (N, d)) + bias[None, :])


def head_v_mixture(seed, b, h, N, d, n_centres, n_outliers, out_lo, out_hi, n_spike=8, centre_norm=4.0,
                   noise=1.0):
    """Mixture of Gaussian centres with token outliers on a few spike channels."""
    rng = _rng(seed, TAG_V, b, h)
    g = _normal(rng, (n_centres, d))
    centres = (centre_norm * g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)
    z = rng.integers(0, n_centres, size=N)
    V = centres[z] + noise * _normal(rng, (N, d))
    toks = rng.choice(N, size=n_outliers, replace=False)
    chans = rng.choice(d, size=n_spike, replace=False)
    if out_lo == out_hi:
        fac = np.full(n_outliers, out_lo, np.float32)
    else:
        fac = rng.uniform(out_lo, out_hi, size=n_outliers).astype(np.float32)
    V[np.ix_(toks, chans)] *= fac[:, None]
    return bf16_bits(V), z.astype(np.int32), centres, np.sort(toks).astype(np.int32)


def drift(V_bits: np.ndarray, seed: int, b: int, h: int, step: int, rel: float = 0.05) -> np.ndarray:
    """V_next = bf16(V + xi * |V|), xi ~ N(0, rel^2) (denoising-step drift)."""
    V = bf16_to_f32(V_bits)
    xi = rel * _normal(_rng(seed, TAG_XI, b, h, step), V.shape)
    return bf16_bits(V + xi * np.abs(V))


def rand_perm(N: int, seed: int, b: int = 0, h: int = 0) -> np.ndarray:
    return _rng(seed, TAG_PERM, b, h).permutation(N).astype(np.int32)


# ------------------------------------------------------------------ workloads
def rope_tables(N: int, d: int, grid=None, base: float = 10000.0):
    """Rotary angle tables (cos, sin), float32 [N, d/2], for tokens in raster order.

    Without `grid`: 1-D positions t with angle t * base^(-2i/d) for pair i. With
    grid = (F, Hh, Ww), F*Hh*Ww = N, a video layout: the channels are split between the
    frame, row and column axes in the proportions a video DiT uses (frame axis
    d - 4*(d//6) channels, each spatial axis 2*(d//6)), and pair i of an axis with c
    channels turns by pos * base^(-2i/c), pos being the token's coordinate on that axis."""
    half = d // 2
    if grid is None:
        pos = np.arange(N, dtype=np.float64)[:, None]
        ang = pos * base ** (-2.0 * np.arange(half)[None, :] / d)
    else:
        F, Hh, Ww = grid
        assert F * Hh * Ww == N
        cs = (d - 4 * (d // 6), 2 * (d // 6), 2 * (d // 6))
        t = np.arange(N)
        coords = (t // (Hh * Ww), (t // Ww) % Hh, t % Ww)
        parts = []
        for c, p in zip(cs, coords):
            parts.append(p[:, None].astype(np.float64) * base ** (-2.0 * np.arange(c // 2)[None, :] / c))
        ang = np.concatenate(parts, axis=1)
        assert ang.shape[1] == half
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# Video grid (frames, rows, columns) of the Wan-shaped workload's 70,400 tokens
WAN_GRID = (22, 40, 80)


WORKLOADS = {
    "tiny": dict(seed=0, B=1, H=1, N=1024, d=128, clusters=8, iters=4, cold=True),
    "expcast": dict(seed=1, B=1, H=8, N=8192, d=128),
    "wan": dict(seed=2, B=1, H=40, N=70400, d=128, clusters=550, iters=2, cold=False),
    "schedule": dict(seed=3, B=1, H=40, N=70400, d=128, clusters=550, steps=20),
    "wan_tight": dict(seed=5, B=1, H=2, N=70400, d=128, clusters=550, iters=2, cold=False),
}
SWEEP = [dict(seed=40 + i, B=1, H=24, N=n, d=128) for i, n in enumerate([16384, 32768, 65536, 131072])] + \
        [dict(seed=44, B=1, H=48, N=32768, d=64)]


def gen_head(kind: str, seed: int, b: int, h: int, N: int, d: int):
    """Q, K, V (bf16 bits, [N, d]) for one head, plus V_prev for 'wan'-type kinds."""
    if kind == "tiny":
        Q = head_q(seed, b, h, N, d)
        K = head_k_biased(seed, b, h, N, d)
        n_out = int(round(0.02 * N))
        V, z, c, toks = head_v_mixture(seed, b, h, N, d, 4, n_out, 20.0, 20.0)
        return dict(Q=Q, K=K, V=V, z_true=z, centres=c, outliers=toks)
    if kind == "expcast":
        Q = head_q(seed, b, h, N, d)
        K = bf16_bits(_normal(_rng(seed, TAG_K, b, h), (N, d)))
        V = bf16_bits(_normal(_rng(seed, TAG_V, b, h), (N, d)))
        return dict(Q=Q, K=K, V=V)
    if kind in ("wan", "sweep", "schedule"):
        Q = head_q(seed, b, h, N, d)
        K = head_k_biased(seed, b, h, N, d)
        n_out = int(round(0.01 * N))
        Vp, z, c, toks = head_v_mixture(seed, b, h, N, d, 64, n_out, 10.0, 30.0)
        V = drift(Vp, seed, b, h, 0)
        return dict(Q=Q, K=K, V=V, V_prev=Vp, z_true=z, centres=c, outliers=toks)
    if kind == "wan_tight":
        Q = head_q(seed, b, h, N, d)
        K = head_k_biased(seed, b, h, N, d)
        n_out = int(round(0.01 * N))
        Vp, z, c, toks = head_v_mixture(seed, b, h, N, d, 64, n_out, 10.0, 30.0, centre_norm=float(np.sqrt(d)),
                                        noise=0.25)
        V = drift(Vp, seed, b, h, 0)
        return dict(Q=Q, K=K, V=V, V_prev=Vp, z_true=z, centres=c, outliers=toks)
    raise ValueError(kind)


def gen(kind: str, heads=None, *, seed=None, B=None, H=None, N=None, d=None):
    """Stacked [B, H', N, d] tensors for the requested heads (default: all)."""
    w = dict(WORKLOADS.get(kind, {}))
    seed = w.get("seed") if seed is None else seed
    B = w.get("B", 1) if B is None else B
    H = w.get("H") if H is None else H
    N = w.get("N") if N is None else N
    d = w.get("d") if d is None else d
    heads = list(range(H)) if heads is None else list(heads)
    out = {}
    for b in range(B):
        for hi, h in enumerate(heads):
            r = gen_head(kind, seed, b, h, N, d)
            for k, v in r.items():
                if k in ("z_true", "centres", "outliers"):
                    continue
                if k not in out:
                    out[k] = np.empty((B, len(heads), N, d), np.uint16)
                out[k][b, hi] = v
    out["meta"] = dict(kind=kind, seed=seed, B=B, H=len(heads), N=N, d=d, heads=heads)
    return out
