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

}  // namespace vc

using namespace vc;

extern "C" int vc_launch_mfma_peak(int grid, int iters, int random_bits, float* out, hipStream_t st) {
  mfma_peak<<<grid, 256, 0, st>>>(iters, random_bits, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
