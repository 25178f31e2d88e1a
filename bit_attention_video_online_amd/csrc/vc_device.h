// vc_device.h -- device helpers shared by the gfx950 kernels of the VC-Attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vc {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kBlock = 128;  // quantisation block and key tile: 128 tokens

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// binary32 -> bfloat16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// exact binary64 value -> bfloat16, one rounding (nearest even), including the
// subnormal range: scale to an integer grid of 8 significant bits and rint.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (x == 0.0) return (uint16_t)(__double_as_longlong(x) >> 48) & 0x8000u;
  int e = ilogb(x);
  if (e < -126) e = -126;
  double q = ldexp(1.0, e - 7);
  double r = rint(x / q) * q;  // x/q and the product are exact (powers of two)
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// neighbouring binary32 value toward +inf (up) or -inf (!up)
__device__ __forceinline__ float f32_step(float f, bool up) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) return __uint_as_float(up ? 1u : 0x80000001u);
  const bool neg = (u >> 31) != 0;
  u = (up != neg) ? u + 1u : u - 1u;
  return __uint_as_float(u);
}

// fl32(S / n) correctly rounded, for an exact binary64 S and integer n >= 1.
// The binary64 quotient is one rounding away from S/n; it only misleads the
// binary32 rounding when it lands exactly on a binary32 midpoint, in which case
// the sign of the exact residual S - q*n decides.
__device__ __forceinline__ float div_to_f32(double S, double n) {
  double q = S / n;
  float f = (float)q;
  uint64_t b = (uint64_t)__double_as_longlong(q);
  if ((b & 0x1fffffffull) == 0x10000000ull && (double)f != q) {
    double r = fma(-q, n, S);
    if (r > 0.0 && (double)f < q) f = f32_step(f, true);
    else if (r < 0.0 && (double)f > q) f = f32_step(f, false);
  }
  return f;
}

// binary32 -> OCP E4M3 byte, round to nearest even. gfx950's v_cvt_pk_fp8_f32 is
// exact RNE for |x| <= 448; callers guarantee |x| <= 448 * (1 + 2^-22) < 464, so
// no value reaches the non-saturating overflow of the instruction.
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xffu;
}
// four bytes at once
__device__ __forceinline__ uint32_t e4m3x4_from_f32(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ExpCast-FP8 bytes (paper page, method step (4)), the exact instruction sequence of the
// attention kernel's hot loop; the elementwise test entry points run these same helpers.
//   t = fma(acc, slope * sigma, fl32(fl32(120 + beta) - slope * m')): one binary32 FMA on the
//       raw score accumulator (slope 8 for E4M3 bytes, 4 for E5M2);
//   byte = cvt_pk_u8_f32(t): round half to even, saturate to [0, 255] (NaN -> 0); four
//       bytes are packed into one dword, byte `sel` replacing that byte of `w`;
//   clamp: a packed per-byte min with 120. It is needed only when some t can reach 120.5,
//       i.e. when fl32(120 + beta) > 120 or |m'| >= 2^16 (the kernel tests this per wave and
//       per key block); below that every byte is already <= 120 and the min is idle.
// Together: clamp(rne(t), 0, 120), since clamping to integer bounds commutes with rounding.
__device__ __forceinline__ float expcast_t(float acc, float slope_sigma, float bias) {
  return __builtin_fmaf(acc, slope_sigma, bias);
}
template <int SEL>
__device__ __forceinline__ uint32_t expcast_cvt(float t, uint32_t w) {
  return __builtin_amdgcn_cvt_pk_u8_f32(t, SEL, w);
}
__device__ __forceinline__ uint32_t expcast_min120(uint32_t w) {  // per-byte min(b, 120)
  uint32_t lo = w & 0x00ff00ffu, hi = (w >> 8) & 0x00ff00ffu;
  lo = min(lo & 0xffffu, 120u) | (min(lo >> 16, 120u) << 16);
  hi = min(hi & 0xffffu, 120u) | (min(hi >> 16, 120u) << 16);
  return lo | (hi << 8);
}
// whether the clamp must run: C0 = fl32(120 + beta), mp the running maximum m' (wave-uniform
// in the kernel). For C0 <= 120 and |m'| < 2^16, t = fma(S, slope sigma, fl32(C0 - slope m'))
// stays below 120.5: S <= max S and m' >= fl32(sigma max S), so slope (sigma S - m') <=
// slope 2^-24 |m'| <= 2^-5 (slope <= 8); fl32(C0 - slope m') is off by at most half an ulp of
// a value below 2^19 + 120, i.e. 2^-5; the FMA's own rounding is below 2^-17.
__device__ __forceinline__ bool expcast_needs_clamp(float C0, float mp) {
  return C0 > 120.0f || fabsf(mp) >= 65536.0f;
}

// Work-group index remap so that consecutive logical tiles share an XCD: the
// hardware deals work-groups round-robin to the 8 XCDs, each with its own L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int nx = 8;
  int x = L % nx, k = L / nx;
  int q = total / nx, r = total % nx;
  return x * q + (x < r ? x : r) + k;
}

}  // namespace vc
