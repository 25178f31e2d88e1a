// vc_peak.hip -- measurement support: the sustained rate of the FP8 matrix core that the
// attention kernel uses (v_mfma_f32_32x32x64_f8f6f4), to set the attention kernel's
// roofline against a measured figure beside the published 5 PFLOP/s dense peak.
//
// Each wave runs `iters` rounds of four independent 32x32x64 FP8 MFMA chains on register
// operands (no memory traffic, no dependency stalls). With `random_bits` the operands are
// per-lane pseudo-random E4M3 patterns, so the multiplier inputs toggle like real data
// (the board's power management reacts to switching activity); otherwise they are fixed
// (A bytes 1.0, B bytes 0.5), so each lane's output sum is exactly 2304 * iters.
// Both E8M0 scales are 127 (2^0).
#include "vc_device.h"

namespace vc {

__global__ __launch_bounds__(256) void mfma_peak(int iters, int random_bits, float* __restrict__ out) {
  v8i a, b;
  uint32_t x = 0x9e3779b9u * (blockIdx.x * 256u + threadIdx.x + 1u);
  for (int k = 0; k < 8; k++) {
    if (random_bits) {
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      a[k] = (int)(x & 0x77777777u);   // finite E4M3 bytes with |value| < 448
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      b[k] = (int)(x & 0x37373737u);
    } else {
      a[k] = 0x38383838;
      b[k] = 0x30303030;
    }
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; it++) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int i = 0; i < 16; i++) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The matrix-core instruction of the attention kernel's score and PV products on caller
// operands, one 32x32x64 tile per wave: D = C + A B^T with A [32 rows][64] and B [32 columns]
// [64] E4M3 codes (both row-major, K fastest) and C, D [32][32] binary32 row-major. Lane l
// supplies row / column l % 32 and K bytes [32 (l / 32), +32) of A and B -- the operand layout
// attn_fwd uses (keys as A rows, queries as B columns) -- and holds accumulator element i at
// row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
__global__ __launch_bounds__(256) void mfma_f8_tiles(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                     const float* __restrict__ C, float* __restrict__ D, int n) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= n) return;
  const int l = threadIdx.x & 63, r = l & 31, h = l >> 5;
  const uint4* pa = reinterpret_cast<const uint4*>(A + (size_t)w * 2048 + r * 64 + 32 * h);
  const uint4* pb = reinterpret_cast<const uint4*>(B + (size_t)w * 2048 + r * 64 + 32 * h);
  const uint4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  v8i a, b;
  a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w; a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
  b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
  v16f c;
  for (int i = 0; i < 16; i++) c[i] = C[(size_t)w * 1024 + (8 * (i >> 2) + 4 * h + (i & 3)) * 32 + r];
  const v16f d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  for (int i = 0; i < 16; i++) D[(size_t)w * 1024 + (8 * (i >> 2) + 4 * h + (i & 3)) * 32 + r] = d[i];
}

}  // namespace vc

using namespace vc;

extern "C" int vc_launch_mfma_f8_tiles(const uint8_t* A, const uint8_t* B, const float* C, float* D, int n,
                                       hipStream_t st) {
  if (n <= 0) return 0;
  mfma_f8_tiles<<<(n + 3) / 4, 256, 0, st>>>(A, B, C, D, n);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int vc_launch_mfma_peak(int grid, int iters, int random_bits, float* out, hipStream_t st) {
  mfma_peak<<<grid, 256, 0, st>>>(iters, random_bits, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
