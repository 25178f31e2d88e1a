"""Helpers shared by the GPU tests: moving seeded numpy inputs onto the device and
running the HIP path through the C ABI binding."""
import numpy as np
import torch

import bit_attention_video_online_amd as vc
import oracle

# The parity contract for the attention output: the oracle's emulation with every score taken in
# the precision of the gfx950 FP8 matrix core (the precision the kernel decides its bytes in) and
# the output rounded once to bfloat16 (the output format).
PARITY = dict(score="gfx950", out_bf16=True)


def emul(q_or, rows, **kw):
    """oracle.attention_emul under the parity contract."""
    return oracle.attention_emul(q_or, rows, **PARITY, **kw)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_quantize(Q, K, V, perm, flags, rope=None):
    """Q, K, V: numpy bf16 bits [B,H,N,d]; perm numpy int32 [B,H,N] or None; rope = (cos, sin)
    float32 [N, d/2] tables or None."""
    B, H, N, d = Q.shape
    out = vc.quantize_outputs(B, H, N, d)
    rc, rs = (None, None) if rope is None else (to_dev(rope[0]), to_dev(rope[1]))
    vc.vc_quantize(to_dev_bf16(Q), to_dev_bf16(K), to_dev_bf16(V), None if perm is None else to_dev(perm), flags, out,
                   rope_cos=rc, rope_sin=rs)
    torch.cuda.synchronize()
    return out


def vq_rowmajor(Vq: np.ndarray) -> np.ndarray:
    """[B,H,nb,d,128] block-transposed codes -> [B,H,N,d] row-major (permuted token order)."""
    B, H, nb, d, T = Vq.shape
    return np.ascontiguousarray(Vq.transpose(0, 1, 2, 4, 3).reshape(B, H, nb * T, d))


def mu_pack_expected(mu_scaled: np.ndarray) -> np.ndarray:
    """Layout of vc_quantize's mu_pack output derived from [nb, d] float32 scaled means:
    [ceil(nb/8), d/32, 2, 64, 8] bf16 bits (MFMA 0: hi in both lane halves; MFMA 1: lo in
    lanes 0-31, zero in lanes 32-63; lane l carries channel 32*block + l%32)."""
    import synth
    nb, d = mu_scaled.shape
    nc = (nb + 7) // 8
    ms = np.zeros((nc * 8, d), np.float32)
    ms[:nb] = mu_scaled
    hi = synth.bf16_bits(ms)
    lo = synth.bf16_bits((ms - synth.bf16_to_f32(hi)).astype(np.float32))
    out = np.zeros((nc, d // 32, 2, 64, 8), np.uint16)
    for c in range(nc):
        for b in range(d // 32):
            for r in range(32):
                ch = 32 * b + r
                out[c, b, 0, r] = hi[8 * c:8 * c + 8, ch]
                out[c, b, 0, 32 + r] = hi[8 * c:8 * c + 8, ch]
                out[c, b, 1, r] = lo[8 * c:8 * c + 8, ch]
    return out


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def mx_unpack(Vq: np.ndarray):
    """MXFP4 layout of vc_quantize's Vq ([B,H,nb,d,128] bytes) -> (codes [B,H,N,d], one E2M1
    code per byte in permuted token order; scales [B,H,nb,d,4] E8M0 bytes)."""
    B, H, nb, d, T = Vq.shape
    flat = Vq.reshape(B, H, nb, d * T)
    codes_b = flat[..., :64 * d].reshape(B, H, nb, d, 64)
    scales = np.ascontiguousarray(flat[..., 64 * d:68 * d].reshape(B, H, nb, d, 4))
    b = np.arange(64)
    q, g, pb = b // 32, (b % 32) // 16, b % 16
    out = np.empty((B, H, nb, 128, d), np.uint8)
    for half in (0, 1):                      # low nibble = even p
        p = 2 * pb + half
        t = 64 * q + 32 * (p // 16) + 16 * g + (p % 16)
        nib = (codes_b >> (4 * half)) & 15    # [B,H,nb,d,64]
        out[:, :, :, t, :] = nib.transpose(0, 1, 2, 4, 3)
    return out.reshape(B, H, nb * 128, d), scales
