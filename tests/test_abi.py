"""C-ABI checks that need no GPU: the library loads, exports every function that
include/vc.h declares, and rejects invalid arguments on the host before anything is
enqueued (the pointers below are never dereferenced: validation fails first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc.h")

vc = pytest.importorskip("bit_attention_video_online_amd")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:vc_status|size_t|int|const char\*)\s+(vc_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vc.LIB_PATH):
        pytest.skip("libvc.so not built")
    return vc.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.vc_abi_version() == 2
    for s in range(8):
        assert vc.vc_status_string(s).startswith(("VC_OK", "VC_E_"))
    assert vc.vc_status_string(99) == "unknown vc_status"


FAKE = ctypes.c_void_p(4096)  # aligned, never dereferenced


def _quant(L, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, perm=None, B=1, H=1, N=256, d=128, block=128, flags=3,
             Qq=ctypes.c_void_p(1 << 20), sQ=ctypes.c_void_p(2 << 20), Kq=ctypes.c_void_p(3 << 20),
             sK=ctypes.c_void_p(4 << 20), Vq=ctypes.c_void_p(5 << 20), sV=ctypes.c_void_p(6 << 20),
             mu=ctypes.c_void_p(7 << 20), mus=ctypes.c_void_p(8 << 20), mup=ctypes.c_void_p(10 << 20),
             ws=ctypes.c_void_p(9 << 20),
             wsb=1 << 30, st=None)
    a.update(kw)
    return L.vc_quantize(a["Q"], a["K"], a["V"], a["perm"], a["B"], a["H"], a["N"], a["d"], a["block"], a["flags"],
                         a["Qq"], a["sQ"], a["Kq"], a["sK"], a["Vq"], a["sV"], a["mu"], a["mus"], a["mup"], a["ws"],
                         a["wsb"],
                         a["st"])


def _quant_rope(L, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, perm=None, rc=ctypes.c_void_p(11 << 20), rs=ctypes.c_void_p(12 << 20), B=1, H=1,
             N=256, d=128, block=128, flags=3 | 16,
             Qq=ctypes.c_void_p(1 << 20), sQ=ctypes.c_void_p(2 << 20), Kq=ctypes.c_void_p(3 << 20),
             sK=ctypes.c_void_p(4 << 20), Vq=ctypes.c_void_p(5 << 20), sV=ctypes.c_void_p(6 << 20),
             mu=ctypes.c_void_p(7 << 20), mus=ctypes.c_void_p(8 << 20), mup=ctypes.c_void_p(10 << 20),
             ws=ctypes.c_void_p(9 << 20), wsb=1 << 30, st=None)
    a.update(kw)
    return L.vc_quantize_rope(a["Q"], a["K"], a["V"], a["perm"], a["rc"], a["rs"], a["B"], a["H"], a["N"], a["d"],
                              a["block"], a["flags"], a["Qq"], a["sQ"], a["Kq"], a["sK"], a["Vq"], a["sV"], a["mu"],
                              a["mus"], a["mup"], a["ws"], a["wsb"], a["st"])


def test_quantize_rope_rejects_bad_arguments(L):
    assert _quant_rope(L, rc=None) == 1
    assert _quant_rope(L, rs=None) == 1
    assert _quant_rope(L, N=200) == 2
    assert _quant_rope(L, flags=64) == 3
    assert _quant_rope(L, rs=ctypes.c_void_p((12 << 20) + 4)) == 5          # misaligned table
    assert _quant_rope(L, rc=ctypes.c_void_p((1 << 20) + 256)) == 7         # table inside an output


def test_quantize_rejects_bad_arguments(L):
    assert _quant(L, Q=None) == 1
    assert _quant(L, N=200) == 2          # not a multiple of 128
    assert _quant(L, N=0) == 2
    assert _quant(L, d=96) == 2
    assert _quant(L, block=64) == 2
    assert _quant(L, B=0) == 2
    assert _quant(L, B=256, H=256, N=128, d=64) == 2   # B*H beyond the 65535 grid limit
    assert _quant(L, flags=64) == 3
    assert _quant(L, wsb=16) == 4
    assert _quant(L, Qq=ctypes.c_void_p((1 << 20) + 4)) == 5   # misaligned
    assert _quant(L, Qq=FAKE) == 7                             # output aliases the inputs


def _attn(L, **kw):
    a = dict(Qq=FAKE, sQ=ctypes.c_void_p(1 << 20), Kq=ctypes.c_void_p(2 << 20), sK=ctypes.c_void_p(3 << 20),
             Vq=ctypes.c_void_p(4 << 20), sV=ctypes.c_void_p(5 << 20), mu=ctypes.c_void_p(6 << 20), B=1, H=1, N=256,
             d=128, block=128, beta=-0.35, flags=4, O=ctypes.c_void_p(7 << 20), st=None)
    a.update(kw)
    return L.vc_attention(a["Qq"], a["sQ"], a["Kq"], a["sK"], a["Vq"], a["sV"], a["mu"], a["B"], a["H"], a["N"], a["d"],
                          a["block"], a["beta"], a["flags"], a["O"], a["st"])


def test_attention_rejects_bad_arguments(L):
    assert _attn(L, O=None) == 1
    assert _attn(L, N=130) == 2
    assert _attn(L, d=32) == 2
    assert _attn(L, beta=float("nan")) == 3
    assert _attn(L, beta=float("inf")) == 3
    assert _attn(L, flags=1 << 8) == 3
    assert _attn(L, flags=8) == 3          # E5M2 bytes exist only as ExpCast
    assert _attn(L, flags=8 | 3) == 3
    assert _attn(L, O=FAKE) == 7
    assert _attn(L, Vq=ctypes.c_void_p((4 << 20) + 8)) == 5


def test_attention_dump_rejects_bad_block(L):
    st = L.vc_attention_dump(FAKE, ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20),
                             ctypes.c_void_p(4 << 20), ctypes.c_void_p(5 << 20), None, 1, 1, 256, 128, 128, -0.35, 4,
                             ctypes.c_void_p(7 << 20), 2, ctypes.c_void_p(8 << 20), None)
    assert st == 3
    st = L.vc_attention_dump(FAKE, ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20),
                             ctypes.c_void_p(4 << 20), ctypes.c_void_p(5 << 20), None, 1, 1, 256, 128, 128, -0.35, 4,
                             ctypes.c_void_p(7 << 20), 0, None, None)
    assert st == 1


def test_cluster_rejects_bad_arguments(L):
    def call(**kw):
        a = dict(V=FAKE, B=1, H=1, N=256, d=128, K=8, iters=2, cold=1, C=ctypes.c_void_p(1 << 20),
                 lab=ctypes.c_void_p(2 << 20), perm=ctypes.c_void_p(3 << 20), ws=ctypes.c_void_p(4 << 20),
                 wsb=1 << 30)
        a.update(kw)
        return L.vc_cluster(a["V"], a["B"], a["H"], a["N"], a["d"], a["K"], a["iters"], a["cold"], a["C"], a["lab"],
                            a["perm"], a["ws"], a["wsb"], None)
    assert call(C=None) == 1
    assert call(N=100) == 2
    assert call(K=0) == 3
    assert call(K=257) == 3          # more clusters than tokens
    assert L.vc_max_clusters() == 8192
    assert call(N=16384, K=8193) == 3  # more clusters than the label histogram holds
    assert call(iters=0) == 3
    assert call(iters=1001) == 3
    assert call(wsb=8) == 4
    assert call(lab=ctypes.c_void_p(3 << 20)) == 7   # labels alias perm


def test_cluster_balanced_rejects_bad_arguments(L):
    def call(**kw):
        a = dict(V=FAKE, B=1, H=1, N=256, d=128, K=8, iters=2, cold=1, lam=0.5, cnt=ctypes.c_void_p(5 << 20),
                 C=ctypes.c_void_p(1 << 20), lab=ctypes.c_void_p(2 << 20), perm=ctypes.c_void_p(3 << 20),
                 ws=ctypes.c_void_p(4 << 20), wsb=1 << 19)
        a.update(kw)
        return L.vc_cluster_balanced(a["V"], a["B"], a["H"], a["N"], a["d"], a["K"], a["iters"], a["cold"], a["lam"],
                                     a["cnt"], a["C"], a["lab"], a["perm"], a["ws"], a["wsb"], None)
    assert call(cnt=None) == 1
    assert call(N=100) == 2
    assert call(K=0) == 3
    assert call(lam=-1.0) == 3
    assert call(lam=float("nan")) == 3
    assert call(lam=float("inf")) == 3
    assert call(wsb=8) == 4
    assert call(cnt=ctypes.c_void_p((5 << 20) + 4)) == 5
    assert call(cnt=ctypes.c_void_p(2 << 20)) == 7    # counts alias labels
    assert call(cnt=ctypes.c_void_p((4 << 20) + 256)) == 7  # counts inside the workspace


def test_workspace_queries(L):
    assert vc.vc_quantize_workspace_bytes(1, 40, 70400, 128) > 0
    assert vc.vc_quantize_workspace_bytes(1, 1, 100, 128) == 0
    assert vc.vc_cluster_workspace_bytes(1, 40, 70400, 128, 550) > 0
    assert vc.vc_cluster_workspace_bytes(1, 1, 256, 128, 300) == 0


def test_debug_expcast_zero_length_is_ok(L):
    assert L.vc_debug_expcast(None, None, None, None, 0, None) == 0
    assert L.vc_debug_expcast(None, None, None, None, 5, None) == 1


def test_debug_mfma_peak_rejects_bad_sizes(L):
    assert L.vc_debug_mfma_peak(1, 1, 0, None, None) == 1
    assert L.vc_debug_mfma_peak(0, 1, 0, ctypes.c_void_p(1 << 20), None) == 3
    assert L.vc_debug_mfma_peak(1, 0, 0, ctypes.c_void_p(1 << 20), None) == 3


def test_debug_expcast_unclamped_and_mfma_tiles_reject_bad_arguments(L):
    assert L.vc_debug_expcast_unclamped(None, None, None, None, 0, None) == 0
    assert L.vc_debug_expcast_unclamped(None, None, None, None, 5, None) == 1
    A, B, C, D = (ctypes.c_void_p(k << 20) for k in (1, 2, 3, 4))
    assert L.vc_debug_mfma_f8(None, None, None, None, 0, None) == 0
    assert L.vc_debug_mfma_f8(None, B, C, D, 1, None) == 1
    assert L.vc_debug_mfma_f8(A, B, C, D, -1, None) == 3
    assert L.vc_debug_mfma_f8(A, B, C, D, (1 << 20) + 1, None) == 3
    assert L.vc_debug_mfma_f8(A, B, C, ctypes.c_void_p((4 << 20) + 4), 1, None) == 5
    assert L.vc_debug_mfma_f8(A, B, C, ctypes.c_void_p((3 << 20) + 1024), 1, None) == 7   # D inside C


def test_valid_calls_need_a_gfx950_device(L):
    """After validation every entry point that would launch checks the current device: with no
    GPU present, valid arguments give VC_E_UNSUPPORTED and nothing runs (this host check is
    skipped where a GPU exists, since there it would launch on the placeholder pointers)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _quant(L) == 5
    assert _attn(L) == 5
    A, B, C, D = (ctypes.c_void_p(k << 20) for k in (1, 2, 3, 4))
    assert L.vc_debug_mfma_f8(A, B, C, D, 1, None) == 5
    assert L.vc_debug_expcast(A, B, C, D, 4, None) == 5
    assert L.vc_debug_mfma_peak(1, 1, 0, ctypes.c_void_p(1 << 20), None) == 5
    assert L.vc_exponent_span(A, 0, 1, 1, 4, 4, B, None) == 5


def test_quantize_noalloc_rejects_bad_arguments(L):
    def call(**kw):
        a = dict(Q=FAKE, K=FAKE, V=FAKE, perm=None, B=1, H=1, N=256, d=128, block=128, flags=3,
                 Qq=ctypes.c_void_p(1 << 20), sQ=ctypes.c_void_p(2 << 20), Kq=ctypes.c_void_p(3 << 20),
                 sK=ctypes.c_void_p(4 << 20), Vq=ctypes.c_void_p(5 << 20), sV=ctypes.c_void_p(6 << 20),
                 mu=ctypes.c_void_p(7 << 20), mus=ctypes.c_void_p(8 << 20), mup=ctypes.c_void_p(10 << 20))
        a.update(kw)
        return L.vc_quantize_noalloc(a["Q"], a["K"], a["V"], a["perm"], a["B"], a["H"], a["N"], a["d"], a["block"],
                                     a["flags"], a["Qq"], a["sQ"], a["Kq"], a["sK"], a["Vq"], a["sV"], a["mu"],
                                     a["mus"], a["mup"], None)
    assert call(Q=None) == 1
    assert call(N=200) == 2
    assert call(flags=64) == 3
    # beyond the 64 MiB scratch: B*H*(N/128)*d = 40 * 1024 * 128 elements need 110 MiB
    assert call(B=1, H=40, N=131072) == 4
    assert call(Qq=ctypes.c_void_p((1 << 20) + 4)) == 5
    assert call(Qq=FAKE) == 7


def test_cluster_incremental_rejects_bad_arguments(L):
    def call(**kw):
        a = dict(V=FAKE, B=1, H=1, N=256, d=128, K=8, decay=0.5, assign=1, C=ctypes.c_void_p(1 << 20),
                 M=ctypes.c_void_p(5 << 20), lab=ctypes.c_void_p(2 << 20), perm=ctypes.c_void_p(3 << 20),
                 ws=ctypes.c_void_p(4 << 20), wsb=1 << 19)
        a.update(kw)
        return L.vc_cluster_incremental(a["V"], a["B"], a["H"], a["N"], a["d"], a["K"], ctypes.c_float(a["decay"]),
                                        a["assign"], a["C"], a["M"], a["lab"], a["perm"], a["ws"], a["wsb"], None)
    assert call(M=None) == 1
    assert call(N=100) == 2
    assert call(K=0) == 3
    assert call(decay=-0.1) == 3
    assert call(decay=1.5) == 3
    assert call(decay=float("nan")) == 3
    assert call(wsb=8) == 4
    assert call(M=ctypes.c_void_p((5 << 20) + 4)) == 5
    assert call(M=ctypes.c_void_p(2 << 20)) == 7        # mass aliases labels


def test_exponent_span_rejects_bad_arguments(L):
    def call(**kw):
        a = dict(X=ctypes.c_void_p(1 << 20), kind=0, B=1, H=2, rows=64, d=128, out=ctypes.c_void_p(2 << 20))
        a.update(kw)
        return L.vc_exponent_span(a["X"], a["kind"], a["B"], a["H"], a["rows"], a["d"], a["out"], None)
    assert call(X=None) == 1
    assert call(out=None) == 1
    assert call(kind=3) == 3
    assert call(kind=-1) == 3
    assert call(rows=0) == 2
    assert call(d=0) == 2
    assert call(B=1 << 16, H=1 << 10, rows=32, d=1) == 2         # 2^31 elements
    assert call(B=256, H=256, rows=1, d=1) == 2                   # B*H above the grid limit
    assert call(X=ctypes.c_void_p((1 << 20) + 1)) == 5            # bf16 needs 2-byte alignment
    assert call(kind=1, X=ctypes.c_void_p((1 << 20) + 2)) == 5    # binary32 needs 4
    assert call(out=ctypes.c_void_p((2 << 20) + 2)) == 5
    assert call(out=ctypes.c_void_p((1 << 20) + 64)) == 7         # out inside X
