"""CPU oracle for the VC-Attention hot path.

TEST INFRASTRUCTURE ONLY: only the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code with
the HIP library and never imports it.

Two parts (paper: "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
Attention", arXiv 2609.15810):

* ``attention_exact`` -- the plain definition O = softmax(Q K^T / sqrt(d)) V in
  binary64 (study-notes page, section 1-1).
* the bit-level emulation of the quantised pipeline: ``kmeans`` (paper page,
  method step (1)), ``quantize`` (step (2)), ``attention_emul`` (steps (3) and
  (4)). The arithmetic lives in ``vc_oracle.c``; this module only marshals arrays.

Every array here is one (batch, head) slice in row-major ``[N, d]`` order;
bf16 tensors are passed as their raw ``uint16`` bit patterns.

Parity status of each function is listed in ``PINS`` below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from decimal import Decimal, getcontext

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_KSMOOTH = 1
FLAG_VSMOOTH = 2
FLAG_HADAMARD = 16
FLAG_MXFP4 = 32
MODE_EXPCAST = 0
MODE_EXP_THEN_CAST = 1
MODE_EXACT_PROB = 2
MODE_EXPCAST_E5M2 = 3
# ExpCast offsets: the pages print -0.35 for E4M3; for E5M2 (an extension the paper page's
# future directions name) the same minimax centring of the mantissa error
# eps2(m) = m - 4 log2(1 + m/4) over m in [0, 4) gives -0.172, taken to two digits.
BETA_E4M3 = -0.35
BETA_E5M2 = -0.17
BLOCK = 128

# which test pins each oracle function (tests/test_oracle_*.py)
PINS = {
    "e4m3_decode/encode": "exhaustive 256-code table from the format definition; log-affine byte property",
    "expcast": "closed-form per-octave agreement 79.61/15.80/4.58 %; TV bound 3.637 %",
    "kmeans_assign": "brute force with Python integers on tiny inputs",
    "kmeans_update": "exact rational means with fractions on tiny inputs",
    "stable_argsort": "numpy.argsort(kind='stable')",
    "quantize": "exactly representable constructions (codes, scales, means reproduced exactly)",
    "attention_emul": "identity-quantiser special case equals exact attention; "
                      "permutation invariance; mean restoration; brute-force scores",
    "attention_exact": "permutation invariance; direct numpy evaluation on tiny inputs",
}


def build(force: bool = False, sanitize_to: str | None = None) -> str:
    """Compile vc_oracle.c into liboracle.so (gcc, OpenMP, no FP contraction). With
    sanitize_to, build an AddressSanitizer + UndefinedBehaviorSanitizer copy at that path
    instead (loaded through VC_ORACLE_LIB with the gcc ASan runtime preloaded)."""
    if sanitize_to:
        cmd = ["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-o", sanitize_to, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        return sanitize_to
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(os.environ.get("VC_ORACLE_LIB") or build())
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        F = ctypes.c_float
        _lib.or_e4m3_decode.restype = ctypes.c_double
        _lib.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib.or_e4m3_encode.restype = ctypes.c_uint8
        _lib.or_e4m3_encode.argtypes = [F]
        _lib.or_e4m3_encode_array.argtypes = [P, P, L]
        _lib.or_e4m3_decode_array.argtypes = [P, P, L]
        _lib.or_e5m2_decode_array.argtypes = [P, P, L]
        _lib.or_e2m1_decode.restype = ctypes.c_double
        _lib.or_e2m1_decode.argtypes = [ctypes.c_uint8]
        _lib.or_e2m1_encode.restype = ctypes.c_uint8
        _lib.or_e2m1_encode.argtypes = [ctypes.c_double]
        _lib.or_expcast.restype = ctypes.c_uint8
        _lib.or_expcast.argtypes = [F, F, F]
        _lib.or_expcast_array.argtypes = [P, P, P, P, L]
        _lib.or_kmeans_assign.argtypes = [P, I, I, P, I, P]
        _lib.or_stable_argsort.argtypes = [P, I, I, P]
        _lib.or_kmeans_update.argtypes = [P, I, I, P, I, P]
        _lib.or_kmeans.argtypes = [P, I, I, I, I, I, P, P, P]
        _lib.or_kmeans_assign_biased.argtypes = [P, I, I, P, I, P, P]
        _lib.or_kmeans_balanced.argtypes = [P, I, I, I, I, I, ctypes.c_float, P, P, P, P]
        _lib.or_kmeans_incremental.argtypes = [P, I, I, I, F, I, P, P, P, P]
        _lib.or_kmeans_cost.restype = ctypes.c_double
        _lib.or_kmeans_cost.argtypes = [P, I, I, P, I, P]
        _lib.or_quantize.restype = I
        _lib.or_quantize.argtypes = [P, P, P, P, I, I, I, F, P, P, P, P, P, P, P, P, P]
        _lib.or_quantize_ex.argtypes = [P, P, P, P, P, P, I, I, I, F, P, P, P, P, P, P, P, P, P, P]
        _lib.or_rope.argtypes = [P, P, P, I, I, P]
        _lib.or_fwht_rows.argtypes = [P, I, I]
        _lib.or_attention_emul.argtypes = [P, P, P, P, P, P, P, I, I, F, I, I, P, P, I, P, P, P, P, I]
        _lib.or_mfma_f8_dot64.restype = F
        _lib.or_mfma_f8_dot64.argtypes = [P, P, F]
        _lib.or_mfma_f8_dot64_array.argtypes = [P, P, P, P, L]
        _lib.or_bf16_from_f64_array.argtypes = [P, P, L]
        _lib.or_attention_exact.argtypes = [P, P, P, I, I, I, P, P]
        _lib.or_exact_mean.restype = ctypes.c_double
        _lib.or_exact_mean.argtypes = [P, L, I]
        _lib.or_exact_sqdist_cmp.restype = I
        _lib.or_exact_sqdist_cmp.argtypes = [P, P, P, I]
        _lib.or_num_threads.restype = I
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().or_num_threads())


# ---------------------------------------------------------------- constants
def log2e_over_sqrt_d(d: int) -> np.float32:
    """c_L = fl32(log2(e) / sqrt(d)), from a 50-digit decimal evaluation."""
    getcontext().prec = 50
    v = (Decimal(1) / Decimal(2).ln()) / Decimal(d).sqrt()
    return np.float32(float(v))  # the double carries > 50 bits; one more rounding to binary32


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- E4M3 and ExpCast
def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().or_e4m3_decode_array(_p(c), _p(out), c.size)
    return out


def e5m2_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().or_e5m2_decode_array(_p(c), _p(out), c.size)
    return out


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    return np.vectorize(lambda v: lib().or_e2m1_decode(int(v)), otypes=[np.float64])(c)


def e2m1_encode(x) -> np.ndarray:
    a = np.asarray(x, np.float64)
    return np.vectorize(lambda v: lib().or_e2m1_encode(float(v)), otypes=[np.uint8])(a)


def e4m3_encode(x) -> np.ndarray:
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().or_e4m3_encode_array(_p(a), _p(out), a.size)
    return out


def expcast(acc, scale8, bias) -> np.ndarray:
    """c = clamp(rne(fma32(acc, scale8, bias)), 0, 120) elementwise (broadcasting)."""
    acc, scale8, bias = np.broadcast_arrays(np.asarray(acc, np.float32), np.asarray(scale8, np.float32),
                                            np.asarray(bias, np.float32))
    a, s, b = _c(acc, np.float32), _c(scale8, np.float32), _c(bias, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().or_expcast_array(_p(a), _p(s), _p(b), _p(out), a.size)
    return out


def mfma_f8_dot64(a, b, c) -> np.ndarray:
    """D = C + sum_k a_k b_k per row, as gfx950's FP8 32x32x64 matrix-core instruction
    accumulates it: a, b uint8 E4M3 codes [..., 64], c binary32 [...]."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    assert a.shape == b.shape and a.shape[-1] == 64
    cc = _c(np.broadcast_to(np.asarray(c, np.float32), a.shape[:-1]), np.float32)
    out = np.empty(a.shape[:-1], np.float32)
    lib().or_mfma_f8_dot64_array(_p(a), _p(b), _p(cc), _p(out), out.size)
    return out


def bf16_round(x) -> np.ndarray:
    """binary64 -> bfloat16 bit patterns, one rounding to nearest even."""
    a = _c(x, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().or_bf16_from_f64_array(_p(a), _p(out), a.size)
    return out


# ---------------------------------------------------------------- k-means
def kmeans_assign(V_bits: np.ndarray, chat: np.ndarray) -> np.ndarray:
    V = _c(V_bits, np.uint16)
    C = _c(chat, np.float32)
    N, d = V.shape
    labels = np.empty(N, np.int32)
    lib().or_kmeans_assign(_p(V), N, d, _p(C), C.shape[0], _p(labels))
    return labels


def stable_argsort(labels: np.ndarray, K: int) -> np.ndarray:
    z = _c(labels, np.int32)
    perm = np.empty(z.shape[0], np.int32)
    lib().or_stable_argsort(_p(z), z.shape[0], K, _p(perm))
    return perm


def kmeans_update(V_bits: np.ndarray, labels: np.ndarray, C: np.ndarray) -> np.ndarray:
    V = _c(V_bits, np.uint16)
    z = _c(labels, np.int32)
    Cn = np.array(C, dtype=np.float32, copy=True, order="C")
    N, d = V.shape
    lib().or_kmeans_update(_p(V), N, d, _p(z), Cn.shape[0], _p(Cn))
    return Cn


def kmeans(V_bits: np.ndarray, K: int, iters: int, cold: bool, C: np.ndarray | None = None):
    """Lloyd k-means on one head's value tokens. Returns (labels, perm, centroids)."""
    V = _c(V_bits, np.uint16)
    N, d = V.shape
    Cn = np.zeros((K, d), np.float32) if C is None else np.array(C, dtype=np.float32, copy=True, order="C")
    labels = np.empty(N, np.int32)
    perm = np.empty(N, np.int32)
    lib().or_kmeans(_p(V), N, d, K, iters, 1 if cold else 0, _p(Cn), _p(labels), _p(perm))
    return labels, perm, Cn


def kmeans_assign_biased(V_bits: np.ndarray, chat: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """argmin_k ||v - chat_k||^2 + bias_k per token, exact, ties to the lowest index."""
    V = _c(V_bits, np.uint16)
    C = _c(chat, np.float32)
    N, d = V.shape
    labels = np.empty(N, np.int32)
    lib().or_kmeans_assign_biased(_p(V), N, d, _p(C), C.shape[0], _p(_c(bias, np.float32)), _p(labels))
    return labels


def kmeans_balanced(V_bits: np.ndarray, K: int, iters: int, cold: bool, lam: float, counts: np.ndarray,
                    C: np.ndarray | None = None):
    """Size-penalised k-means (distance + fl32(lam * n_k), n_k from the previous assignment).
    Returns (labels, perm, centroids, counts after the last assignment)."""
    V = _c(V_bits, np.uint16)
    N, d = V.shape
    Cn = np.zeros((K, d), np.float32) if C is None else np.array(C, dtype=np.float32, copy=True, order="C")
    cnt = np.array(counts, dtype=np.int32, copy=True, order="C")
    assert cnt.shape == (K,)
    labels = np.empty(N, np.int32)
    perm = np.empty(N, np.int32)
    lib().or_kmeans_balanced(_p(V), N, d, K, iters, 1 if cold else 0, ctypes.c_float(lam), _p(cnt), _p(Cn),
                             _p(labels), _p(perm))
    return labels, perm, Cn, cnt


# ---------------------------------------------------------------- quantiser
def rope(x_bits, cos_t, sin_t) -> np.ndarray:
    """RoPE on interleaved channel pairs with binary32 tables [N, d/2]; bf16 result."""
    x = _c(x_bits, np.uint16)
    N, d = x.shape
    out = np.empty_like(x)
    lib().or_rope(_p(x), _p(_c(cos_t, np.float32)), _p(_c(sin_t, np.float32)), N, d, _p(out))
    return out


def fwht_rows(x) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform of every row (binary32, fixed stage order)."""
    a = np.array(x, dtype=np.float32, order="C", copy=True)
    rows, d = a.shape
    lib().or_fwht_rows(_p(a), rows, d)
    return a


def kmeans_incremental(V_bits, C, M, decay: float, assign: bool, labels=None):
    """One cross-step incremental centroid update (see or_kmeans_incremental): returns
    (labels, perm, centroids, masses). Without `assign` the given labels are kept."""
    V = _c(V_bits, np.uint16)
    N, d = V.shape
    Cn = np.array(C, dtype=np.float32, copy=True, order="C")
    Mn = np.array(M, dtype=np.float32, copy=True, order="C")
    K = Cn.shape[0]
    assert Mn.shape == (K,)
    lab = np.zeros(N, np.int32) if labels is None else np.array(labels, dtype=np.int32, copy=True, order="C")
    if not assign and labels is None:
        raise ValueError("kmeans_incremental: labels are required without assign")
    perm = np.empty(N, np.int32)
    lib().or_kmeans_incremental(_p(V), N, d, K, ctypes.c_float(decay), 1 if assign else 0, _p(Cn), _p(Mn),
                                _p(lab), _p(perm))
    return lab, perm, Cn, Mn


def kmeans_cost(V_bits, C, labels) -> float:
    """(1/N) sum_t ||V_t - bf16(C_{z_t})||^2, exact sum, one rounding to binary64."""
    V = _c(V_bits, np.uint16)
    N, d = V.shape
    Cc = _c(C, np.float32)
    return float(lib().or_kmeans_cost(_p(V), N, d, _p(Cc), Cc.shape[0], _p(_c(labels, np.int32))))


def quantize(Q_bits, K_bits, V_bits, perm=None, flags=FLAG_KSMOOTH | FLAG_VSMOOTH, rope_cos=None,
             rope_sin=None) -> dict:
    """Fused quantiser for one head. All outputs row-major; Vq rows are in permuted order.
    With rope_cos/rope_sin ([N, d/2] binary32) Q and K are rotated first; FLAG_HADAMARD
    applies the Q/K Hadamard rotation before quantisation."""
    Q = _c(Q_bits, np.uint16)
    K = _c(K_bits, np.uint16)
    V = _c(V_bits, np.uint16)
    N, d = Q.shape
    nb = N // BLOCK
    pm = None if perm is None else _c(perm, np.int32)
    out = dict(
        Qq=np.empty((N, d), np.uint8), sQ=np.empty(nb, np.float32),
        Kq=np.empty((N, d), np.uint8), sK=np.empty(nb, np.float32),
        Vq=np.empty((N, d), np.uint8), sV=np.empty(d, np.float32),
        mu=np.zeros((nb, d), np.uint16), mu_scaled=np.zeros((nb, d), np.float32),
        kbar=np.empty(d, np.float32),
    )
    if flags & FLAG_MXFP4:
        out["Vs"] = np.empty((nb, d, 4), np.uint8)
    rc_, rs_ = (None, None) if rope_cos is None else (_c(rope_cos, np.float32), _c(rope_sin, np.float32))
    rc = lib().or_quantize_ex(_p(Q), _p(K), _p(V), None if pm is None else _p(pm),
                              None if rc_ is None else _p(rc_), None if rs_ is None else _p(rs_), N, d, int(flags),
                              float(log2e_over_sqrt_d(d)),
                           _p(out["Qq"]), _p(out["sQ"]), _p(out["Kq"]), _p(out["sK"]), _p(out["Vq"]),
                           _p(out["sV"]), _p(out["mu"]), _p(out["mu_scaled"]), _p(out["kbar"]),
                           _p(out["Vs"]) if "Vs" in out else None)
    if rc != 0:
        raise ValueError("oracle quantize: N must be a multiple of 128")
    out["flags"] = flags
    return out


# ---------------------------------------------------------------- attention
def attention_emul(q: dict, rows, beta: float = -0.35, mode: int = MODE_EXPCAST, restore_mean: bool = True,
                   dump_block: int = -1, want_m: bool = False, want_weights: bool = False, score: str = "exact",
                   out_bf16: bool = False):
    """Online-softmax emulation on the given query rows. Returns O [rows, d] (binary64)
    and, when dump_block >= 0, the probability bytes of that key block [rows, 128]; with
    want_m the running max after each key block [rows, N/128]; with want_weights the
    effective weight of every key in the output [rows, N] (keys in the quantised order):
    the decoded probability times 2^(m'_j - m'_final) / l, binary64.

    score: "exact" takes every score as fl32 of the exact dot product of the codes (the
    plain definition); "gfx950" takes it in the precision of the gfx950 FP8 matrix core
    (see or_mfma_f8_dot64 in vc_oracle.c), the precision the attention kernel decides
    its bytes in. out_bf16 rounds O once to bfloat16 (nearest even), the output format,
    and returns it as binary64 values."""
    rows = _c(rows, np.int32)
    N, d = q["Qq"].shape
    O = np.empty((rows.size, d), np.float64)
    dump = np.zeros((rows.size, BLOCK), np.uint8) if dump_block >= 0 else None
    mm = np.zeros((rows.size, N // BLOCK), np.float32) if want_m else None
    W = np.zeros((rows.size, N), np.float64) if want_weights else None
    mu = q["mu_scaled"] if (restore_mean and (q["flags"] & FLAG_VSMOOTH)) else None
    lib().or_attention_emul(_p(q["Qq"]), _p(q["sQ"]), _p(q["Kq"]), _p(q["sK"]), _p(q["Vq"]), _p(q["sV"]),
                            None if mu is None else _p(_c(mu, np.float32)), N, d, float(np.float32(beta)),
                            int(mode), rows.size, _p(rows), _p(O), int(dump_block),
                            None if dump is None else _p(dump), None if mm is None else _p(mm),
                            None if W is None else _p(W), _p(q["Vs"]) if "Vs" in q else None,
                            {"exact": 0, "gfx950": 1}[score])
    if out_bf16:
        O = bf16_bits_to_f32(bf16_round(O)).astype(np.float64)
    res = [O]
    if dump is not None:
        res.append(dump)
    if mm is not None:
        res.append(mm)
    if W is not None:
        res.append(W)
    return res[0] if len(res) == 1 else tuple(res)


def error_terms(Q_bits, K_bits, V_bits, q: dict, perm, rows, beta: float = -0.35, mode: int = MODE_EXPCAST):
    """Split the emulated output's error into a probability term and a value term.

    With P the exact softmax probabilities (binary64 from the bf16 inputs), W the effective
    key weights of the quantised path and V_q the values it actually multiplies
    (s_V * (dec(R_q) + mu/s_V), or s_V * dec(V_q) without V-Smooth), both in the quantised
    key order, O_q - O = (W - P) V + W (V_q - V). Returns the two terms and O_q - O for the
    given rows (each [rows, d]); the terms sum to the third up to binary64 rounding.
    Requires a path whose row sum is the sum of the probabilities it multiplies the values
    by (ExpCast, unquantised probabilities), or no mean restoration (exp-then-cast
    without V-Smooth)."""
    rows = _c(rows, np.int32)
    N, d = q["Qq"].shape
    vs = bool(q["flags"] & FLAG_VSMOOTH)
    if mode == MODE_EXP_THEN_CAST and vs:
        raise ValueError("error_terms: exp-then-cast with mean restoration has two row sums")

    O_q, W = attention_emul(q, rows, beta=beta, mode=mode, want_weights=True)
    order = np.arange(N) if perm is None else np.asarray(perm, np.int64)
    Qf = bf16_bits_to_f32(_c(Q_bits, np.uint16)[rows]).astype(np.float64)
    Kf = bf16_bits_to_f32(_c(K_bits, np.uint16)[order]).astype(np.float64)
    Vf = bf16_bits_to_f32(_c(V_bits, np.uint16)[order]).astype(np.float64)
    s = Qf @ Kf.T / np.sqrt(d)
    P = np.exp(s - s.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    if "Vs" in q:   # MXFP4: E2M1 codes times each group's power-of-two scale
        grp = 2 * (np.arange(BLOCK) >> 6) + ((np.arange(BLOCK) >> 4) & 1)
        sc = np.exp2(q["Vs"].astype(np.float64) - 127.0)                      # [nb, d, 4]
        Vq = e2m1_decode(q["Vq"]) * sc[:, :, grp].transpose(0, 2, 1).reshape(N, d)
    else:
        Vq = e4m3_decode(q["Vq"]).astype(np.float64)
    if vs:
        Vq = Vq + np.repeat(q["mu_scaled"].astype(np.float64), BLOCK, axis=0)
    Vq *= q["sV"].astype(np.float64)[None, :]
    O = P @ Vf
    return (W - P) @ Vf, W @ (Vq - Vf), O_q - O, O


def attention_exact(Q_bits, K_bits, V_bits, rows) -> np.ndarray:
    Q = _c(Q_bits, np.uint16)
    K = _c(K_bits, np.uint16)
    V = _c(V_bits, np.uint16)
    rows = _c(rows, np.int32)
    N, d = Q.shape
    O = np.empty((rows.size, d), np.float64)
    lib().or_attention_exact(_p(Q), _p(K), _p(V), N, d, rows.size, _p(rows), _p(O))
    return O


def pipeline(Q_bits, K_bits, V_bits, rows, *, vsmooth=True, ksmooth=True, expcast_on=True,
             perm=None, beta=-0.35):
    """Full emulated pipeline for one head with a given permutation (None = identity)."""
    flags = (FLAG_KSMOOTH if ksmooth else 0) | (FLAG_VSMOOTH if vsmooth else 0)
    q = quantize(Q_bits, K_bits, V_bits, perm if vsmooth else None, flags)
    mode = MODE_EXPCAST if expcast_on else MODE_EXP_THEN_CAST
    return attention_emul(q, rows, beta=beta, mode=mode), q


# ---------------------------------------------------------------- exact helpers (self-checks)
def exact_mean(x, p: int = 24) -> float:
    a = _c(x, np.float64)
    return float(lib().or_exact_mean(_p(a), a.size, p))


def exact_sqdist_cmp(v, a, b) -> int:
    v, a, b = _c(v, np.float32), _c(a, np.float32), _c(b, np.float32)
    return int(lib().or_exact_sqdist_cmp(_p(v), _p(a), _p(b), v.size))
