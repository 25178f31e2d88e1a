"""VC-Attention hot path on AMD Instinct MI355X (gfx950): thin Python binding.

Every computation runs in the HIP kernels of ``libvc.so`` behind the C ABI declared in
``include/vc.h``; this module only checks tensor metadata, passes raw device pointers
and the current HIP stream, and turns status codes into exceptions. PyTorch is used
for device memory and streams only. There is no CPU fallback: if the library is not
built, importing the functions raises.

Entry points (same names as the C ABI):
  vc_cluster, vc_quantize, vc_attention, vc_attention_dump, vc_debug_expcast,
  vc_debug_expcast_unclamped (as vc_debug_expcast(..., clamp=False)), vc_debug_mfma_f8,
  vc_cluster_workspace_bytes, vc_quantize_workspace_bytes, vc_mu_pack_size, vc_status_string.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# VC_LIB_PATH selects another build of the same library (the CPU suite's host-sanitizer run uses it)
LIB_PATH = os.environ.get("VC_LIB_PATH") or os.path.join(HERE, "libvc.so")

VC_F_KSMOOTH = 1
VC_F_VSMOOTH = 2
VC_F_EXPCAST = 4
VC_F_E5M2 = 8
VC_F_HADAMARD = 16
VC_F_MXFP4 = 32
BLOCK = 128

_STATUS = {0: "VC_OK", 1: "VC_E_NULLPTR", 2: "VC_E_SHAPE", 3: "VC_E_PARAM", 4: "VC_E_WORKSPACE",
           5: "VC_E_UNSUPPORTED", 6: "VC_E_HIP", 7: "VC_E_ALIAS"}


class VCError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvc.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libvc.so not found at %s: run `python bit_attention_video_online_amd/build.py` "
                              "(or __graft_entry__.build()) first" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, U, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
        L.vc_status_string.restype = ctypes.c_char_p
        L.vc_status_string.argtypes = [I]
        L.vc_abi_version.restype = I
        L.vc_cluster_workspace_bytes.restype = S
        L.vc_cluster_workspace_bytes.argtypes = [I, I, I, I, I]
        L.vc_cluster.restype = I
        L.vc_cluster.argtypes = [P, I, I, I, I, I, I, I, P, P, P, P, S, P]
        L.vc_exponent_span.restype = I
        L.vc_exponent_span.argtypes = [P, I, I, I, I, I, P, P]
        L.vc_cluster_balanced.restype = I
        L.vc_cluster_balanced.argtypes = [P, I, I, I, I, I, I, I, ctypes.c_float, P, P, P, P, P, S, P]
        L.vc_quantize_workspace_bytes.restype = S
        L.vc_quantize_workspace_bytes.argtypes = [I, I, I, I, I]
        L.vc_cluster_cost_workspace_bytes.restype = S
        L.vc_cluster_cost_workspace_bytes.argtypes = [I, I, I, I]
        L.vc_cluster_cost.restype = I
        L.vc_cluster_cost.argtypes = [P, P, P, I, I, I, I, I, P, P, S, P]
        L.vc_quantize.restype = I
        L.vc_quantize.argtypes = [P, P, P, P, I, I, I, I, I, U, P, P, P, P, P, P, P, P, P, P, S, P]
        L.vc_quantize_rope.restype = I
        L.vc_quantize_rope.argtypes = [P, P, P, P, P, P, I, I, I, I, I, U, P, P, P, P, P, P, P, P, P, P, S, P]
        L.vc_mu_pack_size.restype = S
        L.vc_mu_pack_size.argtypes = [I, I, I, I]
        L.vc_attention.restype = I
        L.vc_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, U, P, P]
        L.vc_attention_dump.restype = I
        L.vc_attention_dump.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, U, P, I, P, P]
        L.vc_debug_expcast.restype = I
        L.vc_debug_expcast.argtypes = [P, P, P, P, S, P]
        L.vc_debug_expcast_unclamped.restype = I
        L.vc_debug_expcast_unclamped.argtypes = [P, P, P, P, S, P]
        L.vc_cluster_incremental.restype = I
        L.vc_cluster_incremental.argtypes = [P, I, I, I, I, I, F, I, P, P, P, P, P, S, P]
        L.vc_quantize_noalloc.restype = I
        L.vc_quantize_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, U, P, P, P, P, P, P, P, P, P, P]
        L.vc_debug_mfma_f8.restype = I
        L.vc_debug_mfma_f8.argtypes = [P, P, P, P, I, P]
        L.vc_debug_mfma_peak.restype = I
        L.vc_debug_mfma_peak.argtypes = [I, I, I, P, P]
        _lib = L
    return _lib


def vc_status_string(status: int) -> str:
    return lib().vc_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise VCError(status, vc_status_string(status))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU (got %s)" % t.device)
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else ctypes.c_void_p(t.data_ptr() or 16)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dims(x: torch.Tensor):
    if x.dim() != 4:
        raise ValueError("expected [B,H,N,d]")
    return tuple(int(v) for v in x.shape)


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError("%s is required" % name)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s%s, got %s%s" % (name, dtype, tuple(shape), t.dtype, tuple(t.shape)))


# ------------------------------------------------------------------ workspaces
def vc_cluster_workspace_bytes(B, H, N, d, K) -> int:
    return int(lib().vc_cluster_workspace_bytes(B, H, N, d, K))


def vc_mu_pack_size(B, H, N, d) -> int:
    return int(lib().vc_mu_pack_size(B, H, N, d))


def vc_quantize_workspace_bytes(B, H, N, d, block=BLOCK) -> int:
    return int(lib().vc_quantize_workspace_bytes(B, H, N, d, block))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points
def vc_cluster(V, K, iters, cold_start, centroids, labels, perm, ws=None, stream=None):
    """k-means on value tokens; centroids [B,H,K,d] f32 in/out, labels/perm [B,H,N] i32 out."""
    B, H, N, d = _dims(V)
    _need(V, torch.bfloat16, (B, H, N, d), "V")
    _need(centroids, torch.float32, (B, H, K, d), "centroids")
    _need(labels, torch.int32, (B, H, N), "labels")
    _need(perm, torch.int32, (B, H, N), "perm")
    need = vc_cluster_workspace_bytes(B, H, N, d, K)
    if ws is None:
        ws = workspace(need, V.device)
    st = lib().vc_cluster(_ptr(V), B, H, N, d, int(K), int(iters), int(bool(cold_start)), _ptr(centroids),
                          _ptr(labels), _ptr(perm), _ptr(ws), ws.numel(), _stream(stream))
    _check(st)


def vc_cluster_balanced(V, K, iters, cold_start, lam, counts, centroids, labels, perm, ws=None, stream=None):
    """Size-penalised k-means: distances + fl32(lam * n_k); counts [B,H,K] i32 in/out
    (sizes for the first assignment in, sizes after the last one out)."""
    B, H, N, d = _dims(V)
    _need(V, torch.bfloat16, (B, H, N, d), "V")
    _need(counts, torch.int32, (B, H, K), "counts")
    _need(centroids, torch.float32, (B, H, K, d), "centroids")
    _need(labels, torch.int32, (B, H, N), "labels")
    _need(perm, torch.int32, (B, H, N), "perm")
    need = vc_cluster_workspace_bytes(B, H, N, d, K)
    if ws is None:
        ws = workspace(need, V.device)
    st = lib().vc_cluster_balanced(_ptr(V), B, H, N, d, int(K), int(iters), int(bool(cold_start)), float(lam),
                                   _ptr(counts), _ptr(centroids), _ptr(labels), _ptr(perm), _ptr(ws), ws.numel(),
                                   _stream(stream))
    _check(st)


def quantize_outputs(B, H, N, d, device="cuda"):
    nb = N // BLOCK
    kw = dict(device=device)
    return dict(
        Qq=torch.empty((B, H, N, d), dtype=torch.uint8, **kw), sQ=torch.empty((B, H, nb), dtype=torch.float32, **kw),
        Kq=torch.empty((B, H, N, d), dtype=torch.uint8, **kw), sK=torch.empty((B, H, nb), dtype=torch.float32, **kw),
        Vq=torch.empty((B, H, nb, d, BLOCK), dtype=torch.uint8, **kw), sV=torch.empty((B, H, d), dtype=torch.float32, **kw),
        mu=torch.empty((B, H, nb, d), dtype=torch.bfloat16, **kw),
        mu_scaled=torch.empty((B, H, nb, d), dtype=torch.float32, **kw),
        mu_pack=torch.empty((B, H, (nb + 7) // 8, d // 32, 2, 64, 8), dtype=torch.bfloat16, **kw),
    )


def vc_quantize(Q, K, V, perm, flags, out, ws=None, stream=None, block=BLOCK, rope_cos=None, rope_sin=None):
    """Fused quantiser; `out` is a dict as returned by quantize_outputs(). With rope_cos /
    rope_sin (float32 [N, d/2]) Q and K are rotated first (vc_quantize_rope)."""
    B, H, N, d = _dims(Q)
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, (B, H, N, d), n)
    if perm is not None:
        _need(perm, torch.int32, (B, H, N), "perm")
    need = vc_quantize_workspace_bytes(B, H, N, d, block)
    if ws is None:
        ws = workspace(need, Q.device)
    outs = (_ptr(out["Qq"]), _ptr(out["sQ"]), _ptr(out["Kq"]), _ptr(out["sK"]), _ptr(out["Vq"]), _ptr(out["sV"]),
            _ptr(out.get("mu")), _ptr(out.get("mu_scaled")), _ptr(out.get("mu_pack")), _ptr(ws), ws.numel(),
            _stream(stream))
    if rope_cos is None and rope_sin is None:
        st = lib().vc_quantize(_ptr(Q), _ptr(K), _ptr(V), _ptr(perm), B, H, N, d, int(block), int(flags), *outs)
    else:
        _need(rope_cos, torch.float32, (N, d // 2), "rope_cos")
        _need(rope_sin, torch.float32, (N, d // 2), "rope_sin")
        st = lib().vc_quantize_rope(_ptr(Q), _ptr(K), _ptr(V), _ptr(perm), _ptr(rope_cos), _ptr(rope_sin), B, H, N,
                                    d, int(block), int(flags), *outs)
    _check(st)
    return out


def vc_cluster_incremental(V, decay, assign, C, M, labels, perm, ws=None, stream=None):
    """One cross-step incremental centroid update: C float32 [B,H,K,d] and M float32 [B,H,K]
    in/out; labels int32 [B,H,N] out with `assign`, else in; perm int32 [B,H,N] out."""
    B, H, N, d = _dims(V)
    K = C.shape[2]
    _need(V, torch.bfloat16, (B, H, N, d), "V")
    _need(C, torch.float32, (B, H, K, d), "centroids")
    _need(M, torch.float32, (B, H, K), "mass")
    _need(labels, torch.int32, (B, H, N), "labels")
    _need(perm, torch.int32, (B, H, N), "perm")
    if ws is None:
        ws = workspace(vc_cluster_workspace_bytes(B, H, N, d, K), V.device)
    _check(lib().vc_cluster_incremental(_ptr(V), B, H, N, d, K, float(decay), int(bool(assign)), _ptr(C), _ptr(M),
                                        _ptr(labels), _ptr(perm), _ptr(ws), ws.numel(), _stream(stream)))
    return C, M, labels, perm


def vc_quantize_noalloc(Q, K, V, perm, flags, out, stream=None, block=BLOCK):
    """vc_quantize without a workspace: the library's own device scratch serves instead (no
    allocation in the call; calls overlapping on one device race)."""
    B, H, N, d = _dims(Q)
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, torch.bfloat16, (B, H, N, d), n)
    if perm is not None:
        _need(perm, torch.int32, (B, H, N), "perm")
    st = lib().vc_quantize_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(perm), B, H, N, d, int(block), int(flags),
                                   _ptr(out["Qq"]), _ptr(out["sQ"]), _ptr(out["Kq"]), _ptr(out["sK"]),
                                   _ptr(out["Vq"]), _ptr(out["sV"]), _ptr(out.get("mu")), _ptr(out.get("mu_scaled")),
                                   _ptr(out.get("mu_pack")), _stream(stream))
    _check(st)
    return out


def vc_cluster_cost(V, C, labels, cost, ws=None, stream=None):
    """k-means objective per (b,h) into cost (float64 [B,H]): (1/N) sum ||V_t - bf16(C_z)||^2."""
    B, H, N, d = _dims(V)
    K = C.shape[2]
    _need(V, torch.bfloat16, (B, H, N, d), "V")
    _need(C, torch.float32, (B, H, K, d), "centroids")
    _need(labels, torch.int32, (B, H, N), "labels")
    _need(cost, torch.float64, (B, H), "cost")
    if ws is None:
        ws = workspace(int(lib().vc_cluster_cost_workspace_bytes(B, H, N, d)), V.device)
    _check(lib().vc_cluster_cost(_ptr(V), _ptr(C), _ptr(labels), B, H, N, d, K, _ptr(cost), _ptr(ws), ws.numel(),
                                 _stream(stream)))
    return cost


def vc_exponent_span(X, as_bf16=False, stream=None):
    """Exponent range per (b,h) of X ([B,H,rows,d] bf16 or float32; float32 read as the bf16
    value it rounds to with as_bf16): int32 [B,H,2] = (largest exponent, lowest significand
    bit exponent) over the nonzero finite elements; (INT32_MIN, INT32_MAX) for an all-zero head."""
    if X.dim() != 4:
        raise ValueError("X must be [B,H,rows,d]")
    B, H, R, d = X.shape
    if X.dtype == torch.bfloat16:
        kind = 0
    elif X.dtype == torch.float32:
        kind = 2 if as_bf16 else 1
    else:
        raise ValueError("X must be bfloat16 or float32")
    if not X.is_contiguous():
        raise ValueError("X must be contiguous")
    out = torch.empty((B, H, 2), dtype=torch.int32, device=X.device)
    _check(lib().vc_exponent_span(_ptr(X), kind, B, H, R, d, _ptr(out), _stream(stream)))
    return out


def vc_attention(q, O, beta=-0.35, flags=VC_F_EXPCAST, restore_mean=True, stream=None, block=BLOCK):
    """Attention over the quantised tensors `q` (dict from vc_quantize); O bf16 [B,H,N,d]."""
    B, H, N, d = _dims(O)
    mu = q["mu_pack"] if restore_mean else None
    st = lib().vc_attention(_ptr(q["Qq"]), _ptr(q["sQ"]), _ptr(q["Kq"]), _ptr(q["sK"]), _ptr(q["Vq"]), _ptr(q["sV"]),
                            _ptr(mu), B, H, N, d, int(block), float(beta), int(flags), _ptr(O), _stream(stream))
    _check(st)
    return O


def vc_attention_dump(q, O, dump_block, codes, beta=-0.35, flags=VC_F_EXPCAST, restore_mean=True, stream=None,
                      block=BLOCK):
    B, H, N, d = _dims(O)
    _need(codes, torch.uint8, (B, H, N, BLOCK), "codes")
    mu = q["mu_pack"] if restore_mean else None
    st = lib().vc_attention_dump(_ptr(q["Qq"]), _ptr(q["sQ"]), _ptr(q["Kq"]), _ptr(q["sK"]), _ptr(q["Vq"]),
                                 _ptr(q["sV"]), _ptr(mu), B, H, N, d, int(block), float(beta), int(flags), _ptr(O),
                                 int(dump_block), _ptr(codes), _stream(stream))
    _check(st)
    return O, codes


def vc_debug_mfma_peak(grid, iters, random_bits, out, stream=None):
    """Sustained FP8 MFMA measurement kernel; out: float32 [grid * 256] on the device."""
    _need(out, torch.float32, (grid * 256,), "out")
    _check(lib().vc_debug_mfma_peak(int(grid), int(iters), int(bool(random_bits)), _ptr(out), _stream(stream)))
    return out


def vc_debug_expcast(acc, scale8, bias, codes, stream=None, clamp=True):
    """The attention kernel's ExpCast byte sequence elementwise: with clamp (default) its
    clamped path (vc_debug_expcast), else its unclamped path (vc_debug_expcast_unclamped)."""
    n = acc.numel()
    for t, name in ((acc, "acc"), (scale8, "scale8"), (bias, "bias")):
        _need(t, torch.float32, tuple(acc.shape), name)
    _need(codes, torch.uint8, tuple(acc.shape), "codes")
    fn = lib().vc_debug_expcast if clamp else lib().vc_debug_expcast_unclamped
    st = fn(_ptr(acc), _ptr(scale8), _ptr(bias), _ptr(codes), n, _stream(stream))
    _check(st)
    return codes


def vc_debug_mfma_f8(A, B, C, D, stream=None):
    """D = C + A B^T per 32x32x64 tile on the attention kernel's FP8 matrix-core instruction:
    A, B uint8 [n, 32, 64], C, D float32 [n, 32, 32] on the device."""
    n = int(A.shape[0])
    _need(A, torch.uint8, (n, 32, 64), "A")
    _need(B, torch.uint8, (n, 32, 64), "B")
    _need(C, torch.float32, (n, 32, 32), "C")
    _need(D, torch.float32, (n, 32, 32), "D")
    _check(lib().vc_debug_mfma_f8(_ptr(A), _ptr(B), _ptr(C), _ptr(D), n, _stream(stream)))
    return D
