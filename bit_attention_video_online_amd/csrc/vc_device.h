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

// ExpCast-FP8 byte (paper page, method step (4)): the score enters as the raw
// accumulator; t = fma(acc, 8*sigma, fl32(fl32(120+beta) - 8 m')) is one binary32
// FMA, then round half to even and clamp to [0, 120]. med3 clamps in the float
// domain (clamping to integer bounds commutes with rounding) and cvt_pk_u8_f32
// rounds to nearest even; the byte lands in position `sel` of `old`.
// The FMA is written as the instruction itself: the attention kernel also evaluates the
// same FMA on its unclamped fast path, and an opaque instruction keeps the compiler from
// hoisting both into one shared set of 32 live temporaries.
__device__ __forceinline__ uint32_t expcast_byte(float acc, float scale8, float bias, uint32_t old, int sel) {
  float t;
  asm("v_fma_f32 %0, %1, %2, %3" : "=v"(t) : "v"(acc), "v"(scale8), "v"(bias));
  t = __builtin_amdgcn_fmed3f(t, 0.0f, 120.0f);
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_pk_u8_f32(t, 0, old);
    case 1: return __builtin_amdgcn_cvt_pk_u8_f32(t, 1, old);
    case 2: return __builtin_amdgcn_cvt_pk_u8_f32(t, 2, old);
    default: return __builtin_amdgcn_cvt_pk_u8_f32(t, 3, old);
  }
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
