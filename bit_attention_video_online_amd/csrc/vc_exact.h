// vc_exact.h -- exact sums in binary64 pairs for the k-means and quantiser kernels.
//
// The centroid update, the block and key means and the exact k-means distances are
// defined on exact sums of bf16 values (rounded once at the end). A sum s is carried as
// an unevaluated pair hi + lo: every term enters hi through an error-free transformation
// (Knuth's TwoSum; products through the FMA-based TwoProduct) and the rounding error it
// leaves goes to lo. hi + lo is then the exact sum as long as lo's own additions do not
// round, i.e. while every term is an integer multiple of 2^q and the magnitudes of all
// the errors collected in lo stay below 2^(q+53): for n terms below 2^(E+1) that holds
// when E - q <= 103 - 2 ceil(log2 n) (every error is at most 2^-53 of a partial sum, which
// is below n 2^(E+1), and terms plus merges of partial pairs give at most 2n errors). Under that
// condition the result is independent of the order of the terms and of how the partial
// pairs are combined. All arithmetic here is op by op (the library is built without FMA
// contraction), which TwoSum relies on.
#pragma once
#include "vc_device.h"

namespace vc {

// s = fl64(a + b), e = (a + b) - s exactly
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

struct dpair {
  double hi, lo;
};

__device__ __forceinline__ void dp_add(dpair& a, double x) {
  double s, e;
  two_sum(a.hi, x, s, e);
  a.hi = s;
  a.lo += e;
}
// a += x * x (x * x = p + e exactly: TwoProduct with one FMA)
__device__ __forceinline__ void dp_add_sq(dpair& a, double x) {
  const double p = x * x;
  const double e = fma(x, x, -p);
  dp_add(a, p);
  a.lo += e;
}
__device__ __forceinline__ void dp_merge(dpair& a, const dpair& b) {
  double s, e;
  two_sum(a.hi, b.hi, s, e);
  a.hi = s;
  a.lo = (a.lo + b.lo) + e;
}
// the same exact value with hi = fl64(hi + lo) (RNE) and lo the exact remainder: for such
// pairs lexicographic order of (hi, lo) is the order of the exact values
__device__ __forceinline__ dpair dp_norm(const dpair& a) {
  dpair r;
  two_sum(a.hi, a.lo, r.hi, r.lo);
  return r;
}
__device__ __forceinline__ dpair dp_shfl_xor(const dpair& a, int m) {
  return dpair{__shfl_xor(a.hi, m), __shfl_xor(a.lo, m)};
}

// fl32(s / n), nearest even, for the exact pair s and an integer 1 <= n <= 2^26. With
// S = fl64(s), r = s - S and q = fl64(S / n), the binary32 rounding of q is the right one
// unless q lies within two binary64 steps of a binary32 midpoint M next to fl32(q) (q is
// within 1.5 steps of s / n); then the sign of s - M n = fl64(S - M n) + r decides (the
// FMA is exact there: M n and S agree to a few units of their common grid) and an exact
// zero is a tie, resolved to the even neighbour. Subnormal binary32 results included.
__device__ __forceinline__ float dp_div_to_f32(const dpair& s, double n) {
  const dpair a = dp_norm(s);
  const double S = a.hi, r = a.lo;
  if (S == 0.0) return 0.0f;
  const double q = S / n;
  const float f = (float)q;
  const float dn = f32_step(f, false), up = f32_step(f, true);
  const double tol = ldexp(2.0, ilogb(q) - 52);
  const double Mhi = 0.5 * ((double)f + (double)up), Mlo = 0.5 * ((double)f + (double)dn);
  if (fabs(q - Mhi) <= tol) {
    const double t = fma(-Mhi, n, S) + r;
    if (t > 0.0) return up;
    if (t < 0.0) return f;
    return (__float_as_uint(f) & 1u) ? up : f;
  }
  if (fabs(q - Mlo) <= tol) {
    const double t = fma(-Mlo, n, S) + r;
    if (t < 0.0) return dn;
    if (t > 0.0) return f;
    return (__float_as_uint(f) & 1u) ? dn : f;
  }
  return f;
}

// bfloat16 nearest (even) to s * 2^k for the exact pair s (k <= 0, no binary64 underflow):
// with S = fl64(s) and r = s - S, the binary64 value x = S 2^k rounds like the exact one
// unless x is itself a bfloat16 midpoint and r != 0, in which case r's sign decides.
__device__ __forceinline__ uint16_t dp_to_bf16_scaled(const dpair& s, int k) {
  const dpair a = dp_norm(s);
  const double x = ldexp(a.hi, k), rx = ldexp(a.lo, k);
  const uint16_t h = f64_to_bf16(x);
  if (rx == 0.0) return h;
  const float xf = (float)x;
  if ((double)xf != x) return h;  // a bfloat16 midpoint has 9 significant bits
  const uint32_t u = __float_as_uint(xf);
  if ((u & 0xffffu) != 0x8000u) return h;
  const uint16_t below = (uint16_t)(u >> 16);  // magnitude rounded down, sign kept
  const bool away = (x > 0.0) == (rx > 0.0);   // the exact value lies beyond the midpoint
  return away ? (uint16_t)(below + 1u) : below;
}

}  // namespace vc
