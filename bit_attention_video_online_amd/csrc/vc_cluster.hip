// vc_cluster.hip -- online k-means on value tokens for gfx950.
//
// Paper page (paper.rainbus.top), method step (1): each (batch, head) gets labels z
// from a lightweight online k-means over its value tokens and the permutation
// pi = argsort(z); centroids are warm-started across denoising steps. Reading
// taken here: Lloyd iterations (assign to the nearest bf16-rounded centroid by
// squared Euclidean distance, ties to the lowest index; centroid = binary32 rounding
// of the exact member mean; empty clusters keep their centroid); pi is stable.
//
// Kernels, per iteration:
//   cl_prep    chat = bf16(C) (bf16 bits), |chat|^2
//   cl_assign_mfma  distances |c|^2 - 2 v.c with the dot products on bf16 MFMA, a
//              rigorous per-distance error bound, and an exact re-rank (binary64 pairs) of
//              every token whose best candidate is not separated from the rest by the bounds.
//   cl_hist / cl_scan_k / cl_scan_c / cl_scatter   stable counting sort of the labels (pi)
//   cl_update  C_k = fl32(exact sum of members / count), sums as binary64 pairs in pi order
// Size-penalised variant (cheap balancing; the paper page's ablation measures balanced
// k-means and sets it aside for its cost): every distance gets b_k = fl32(lambda n_k),
// n_k the size of cluster k after the previous assignment, folded into |chat_k|^2 by
// cl_prep, so the assignment loop is unchanged; only the certainty bound and the exact
// re-rank take b_k into account.
// No atomics on floating-point data: every result is run-to-run deterministic.
#include "vc_exact.h"

namespace vc {

constexpr int kChunk = 256;   // tokens per sort chunk
constexpr int kMaxClusters = 8192;

__global__ void cl_cold(const uint16_t* __restrict__ V, float* __restrict__ C, int N, int K, int D) {
  const int k = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const long long t = ((long long)(2 * k + 1) * N) / (2LL * K);
  C[((size_t)bh * K + k) * D + c] = bf16_to_f32(V[((size_t)bh * N + t) * D + c]);
}

__global__ void cl_prep(const float* __restrict__ C, uint16_t* __restrict__ chat, float* __restrict__ cnorm, int K,
                        int D, const int32_t* __restrict__ nk, float lam) {
  __shared__ double part[128];
  const int k = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const size_t o = ((size_t)bh * K + k) * D + c;
  const uint16_t hb = f32_to_bf16(C[o]);
  const float h = bf16_to_f32(hb);
  chat[o] = hb;
  part[c] = (double)h * (double)h;  // exact square of a bf16 value
  __syncthreads();
  if (c == 0) {
    double s = 0.0;
    for (int i = 0; i < D; i++) s += part[i];
    if (nk) s += (double)(lam * (float)nk[(size_t)bh * K + k]);  // b_k: one binary32 rounding
    cnorm[(size_t)bh * K + k] = (float)s;
  }
}

// per-token record of one lane group: its three smallest keys, d1 <= d2 <= d3 (the low bits of
// a key are its centroid index)
struct Best {
  float d1, d2, d3;
};

// exact distance (hi, lo) of a re-ranked token and its centroid index
struct Exact {
  double d, lo;
  int k;
};

// Rigorous lower bound of d_k - e_k over every centroid whose computed distance' is >= x
// (x = d2): with |c_k| <= |v| + sqrt(D_k) and D_k <= d_k + e_k + |v|^2, the bound
// e_k <= F(e) = 2(2 gam |v| c(e) + u (c(e)^2 + |x|)), c(e) = |v| + sqrt(x + e + |v|^2),
// is increasing in x, so x - E(x) is increasing too and bounds every other centroid. E is
// taken from above: two steps of F from a crude upper starting value, then doubled.
// With size penalties b_k >= 0 folded into the norms, the rounding term of a norm is
// u (|c_k|^2 + b_k), and b_k <= d_k + e_k + |v|^2 as well (the exact distance' minus
// |v - c_k|^2 - |v|^2 is b_k), so F gains u (x + e + |v|^2); the bound on |c_k| holds
// unchanged since |v - c_k|^2 <= d_k + e_k + |v|^2 still.
__device__ __forceinline__ double others_lower_bound(double x, double vn, double gam, double u, bool biased) {
  auto F = [&](double e) {
    const double c = vn + sqrt(fmax(x + e + vn * vn, 0.0));
    const double b = biased ? fmax(x + e + vn * vn, 0.0) : 0.0;
    return 2.0 * (2.0 * gam * vn * c + u * (c * c + b + fabs(x)));
  };
  const double e0 = 0.5 * (fabs(x) + vn * vn) + 1.0;
  const double e1 = F(e0);
  if (!(e1 <= e0)) return -__builtin_inf();  // the crude start was not above the fixed point
  return x - 2.0 * F(e1);
}

// ---------------------------------------------------------------------------
// Assignment on the matrix cores. S^T = chat V^T with v_mfma_f32_16x16x32_bf16: the
// bf16 products are exact and the accumulation error of the instruction chain was
// measured at <= 2^-21.3 sum|v_c chat_c| on adversarial wide-range data, far inside
// the binary32 recursive-summation bound gamma_d sum|v_c chat_c| used below (doubled),
// so the same certainty test and exact re-rank apply.
// Work-group: 4 waves x 64 tokens (four 16-token groups), so every staged centroid chunk
// serves 256 tokens. Centroid chunks of 64 rows of
// bf16 are staged in LDS with a padded row stride (conflict-free 16-byte fragment
// reads). Per MFMA the lane holds one token (lane % 16) and four centroids
// (4 * (lane / 16) + i); the four lane groups of a token are merged at the end.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAssignTokens = 256;  // tokens per assignment work-group

template <int D>
__global__ __launch_bounds__(256) void cl_assign_mfma(const uint16_t* __restrict__ V, const uint16_t* __restrict__ chat,
                                                      const float* __restrict__ cnorm, int N, int K,
                                                      int32_t* __restrict__ labels, const int32_t* __restrict__ nk,
                                                      float lam) {
  constexpr int KS = D / 32;            // MFMA k-steps over the feature dimension
  constexpr int ROWB = 2 * D + 16;      // padded LDS row stride (bytes)
  constexpr int CCH = 64;               // centroids per chunk
  constexpr int NG = kAssignTokens / 64; // 16-token groups per wave
  __shared__ __attribute__((aligned(16))) uint8_t Cs[CCH * ROWB];
  __shared__ float cn_s[CCH];
  __shared__ float vn_s[kAssignTokens];
  __shared__ Best rec[kAssignTokens][4];
  __shared__ int unsure[kAssignTokens];
  constexpr int RB = 64;  // uncertain tokens per re-rank batch
  __shared__ Exact rr[RB][4];
  __shared__ int n_unsure;

  const int bh = blockIdx.y, t0 = blockIdx.x * kAssignTokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, lg = lane >> 4;
  const uint16_t* Vh = V + (size_t)bh * N * D;
  const uint16_t* Ch = chat + (size_t)bh * K * D;
  const float* Nh = cnorm + (size_t)bh * K;

  // token fragments (B operand): token row, features [32 ks + 8 lg, +8)
  bf16x8 vb[NG][KS];
  float vn[NG];
  for (int g = 0; g < NG; g++) {
    const int t = min(t0 + wave * 16 * NG + g * 16 + r16, N - 1);  // tokens past N repeat the last
    float s = 0.0f;
    for (int ks = 0; ks < KS; ks++) {
      uint4 raw = *reinterpret_cast<const uint4*>(Vh + (size_t)t * D + 32 * ks + 8 * lg);
      memcpy(&vb[g][ks], &raw, 16);
      uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      for (int q = 0; q < 4; q++) {
        float lo = __uint_as_float(w[q] << 16), hi = __uint_as_float(w[q] & 0xffff0000u);
        s = __builtin_fmaf(lo, lo, s);
        s = __builtin_fmaf(hi, hi, s);
      }
    }
    // |v|^2 = sum over the four lane groups of this token
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    vn[g] = sqrtf(s) * 1.0001f;  // upper bound of |v|
    if (lg == 0) vn_s[wave * 16 * NG + g * 16 + r16] = vn[g];
  }
  const float u = 5.9604645e-8f;  // 2^-24
  const float gam = (float)D * u / (1.0f - (float)D * u);
  // Every computed distance' d_k is within e_k = 2(2 gamma |v||c_k| + u(|c_k|^2 + |d_k|))
  // of its exact value (bf16 products are exact; the accumulation error is inside the
  // binary32 bound). Keys: d_k with the low kbits bits of its binary32 pattern replaced by k
  // (the centroid count rounded up to whole chunks fits in kbits), so |key_k - d_k| <=
  // 2^(kbits-23) |d_k| + 2^(kbits-149) (the exponent field is untouched) and the keys of
  // different centroids differ. Per token and lane group the loop keeps, branch-free, the
  // three smallest keys (three medians of three per distance). At the end, with x1 >= the
  // best centroid's d and x2 (x3) <= every d_k whose key is at least the second (third)
  // smallest: others_lower_bound(x2) > x1 + e1 proves the best index exact; otherwise
  // others_lower_bound(x3) > x1 + e1 proves the exact argmin is one of the two smallest keys,
  // whose two exact distances decide; otherwise the token goes to the full exact re-rank.
  // Near ties (within the key perturbation) always fall to an exact comparison.
  const int kpad = (K + 63) / 64 * 64;
  const int kbits = 32 - __clz(kpad - 1);
  const uint32_t kmask = (1u << kbits) - 1u;
  // -inf as an operand the compiler cannot see: median(d1, key, -inf) is min(d1, key), which
  // it would otherwise rewrite into a NaN-canonicalising max and a min (two instructions)
  float ninf;
  asm volatile("s_mov_b32 %0, 0xff800000" : "=s"(ninf));
  float d1[NG], d2[NG], d3[NG];
  for (int g = 0; g < NG; g++) {
    d1[g] = __builtin_inff(); d2[g] = __builtin_inff(); d3[g] = __builtin_inff();
  }
  const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  // centroid chunks of CCH bf16 rows go through registers into LDS; the next chunk's global
  // loads are issued before the current chunk is ranked, so their latency is hidden
  constexpr int SPT = CCH * (D / 8) / 256;  // 16-byte pieces per thread per chunk
  uint4 pre[SPT];
  float pre_cn = 3.0e38f;
  auto load_chunk = [&](int k0) {
    for (int p = 0; p < SPT; p++) {
      const int i = tid + 256 * p;
      const int k = i / (D / 8), c8 = (i % (D / 8)) * 8;
      pre[p] = make_uint4(0, 0, 0, 0);
      if (k0 + k < K) pre[p] = *reinterpret_cast<const uint4*>(Ch + (size_t)(k0 + k) * D + c8);
    }
    // padding past K gets zero rows and a huge finite norm, so its distance never wins
    if (tid < CCH) pre_cn = (k0 + tid < K) ? Nh[k0 + tid] : 3.0e38f;
  };
  load_chunk(0);
  for (int k0 = 0; k0 < K; k0 += CCH) {
    __syncthreads();
    // stage chat rows [k0, k0+64) (bf16)
    for (int p = 0; p < SPT; p++) {
      const int i = tid + 256 * p;
      const int k = i / (D / 8), c8 = (i % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(Cs + k * ROWB + 2 * c8) = pre[p];
    }
    if (tid < CCH) cn_s[tid] = pre_cn;
    __syncthreads();
    if (k0 + CCH < K) load_chunk(k0 + CCH);
    for (int cb = 0; cb < CCH / 16; cb++) {
      v4f acc[NG];
      for (int g = 0; g < NG; g++) acc[g] = zero4;
      for (int ks = 0; ks < KS; ks++) {
        bf16x8 a;
        memcpy(&a, Cs + (16 * cb + r16) * ROWB + 2 * (32 * ks + 8 * lg), 16);
        for (int g = 0; g < NG; g++) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vb[g][ks], acc[g], 0, 0, 0);
      }
      for (int i = 0; i < 4; i++) {
        const int kl = 16 * cb + 4 * lg + i;
        const float cnk = cn_s[kl];
        const uint32_t kk = (uint32_t)(k0 + kl);
        for (int g = 0; g < NG; g++) {
          const float dd = __builtin_fmaf(-2.0f, acc[g][i], cnk);  // exact scaling, one rounding
          float key;  // (bits(dd) & ~kmask) | k as one v_and_or_b32 (the compiler splits it in two)
          asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(key) : "v"(dd), "s"(~kmask), "v"(kk));
          // d1 <= d2 <= d3 always: the new third is the median of (d2, d3, key), the new second
          // that of (d1, d2, key), the new best that of (d1, key, -inf)
          d3[g] = __builtin_amdgcn_fmed3f(d2[g], d3[g], key);
          d2[g] = __builtin_amdgcn_fmed3f(d1[g], d2[g], key);
          d1[g] = __builtin_amdgcn_fmed3f(d1[g], key, ninf);
        }
      }
    }
  }
  // merge the four lane groups of each token through LDS
  if (tid == 0) n_unsure = 0;
  for (int g = 0; g < NG; g++) rec[wave * 16 * NG + g * 16 + r16][lg] = Best{d1[g], d2[g], d3[g]};
  __syncthreads();
  const int32_t* nkh = nk ? nk + (size_t)bh * K : nullptr;
  auto better = [](double d2, double l2, int k2, double d, double l, int k) {
    return d2 < d || (d2 == d && (l2 < l || (l2 == l && k2 < k)));
  };
  // normalised exact distance pair plus the size penalty b_k = fl32(lam n_k), normalised again
  auto with_bias = [&](const dpair& d, int k) {
    if (!nkh) return d;
    double h, e;
    two_sum(d.hi, (double)(lam * (float)nkh[k]), h, e);
    return dp_norm(dpair{h, d.lo + e});
  };
  if (tid < kAssignTokens && t0 + tid < N) {
    float a1 = rec[tid][0].d1, a2 = rec[tid][0].d2, a3 = rec[tid][0].d3;  // the three smallest keys
    auto insert = [&](float x) {  // keys are distinct, so the sorted triple stays exact
      a3 = __builtin_amdgcn_fmed3f(a2, a3, x);
      a2 = __builtin_amdgcn_fmed3f(a1, a2, x);
      a1 = fminf(a1, x);
    };
    for (int x = 1; x < 4; x++) { insert(rec[tid][x].d1); insert(rec[tid][x].d2); insert(rec[tid][x].d3); }
    const int k1 = (int)(__float_as_uint(a1) & kmask), k2 = (int)(__float_as_uint(a2) & kmask);
    int label = -1;  // -1: full re-rank
    if ((unsigned)k1 < (unsigned)K) {
      const double vn = vn_s[tid], dg = (double)gam, du = (double)u;
      const double delta = ldexp(1.0, kbits - 23), eta = ldexp(1.0, kbits - 149);
      const double y1 = a1, y2 = a2, y3 = a3;
      const double x1 = y1 + delta * fabs(y1) + eta;  // >= the best centroid's distance'
      const double x2 = y2 - delta * fabs(y2) - eta;  // <= the distance' of every other centroid
      const double x3 = y3 - delta * fabs(y3) - eta;  // <= that of every centroid but the first two
      const double cnk = Nh[k1], ck = sqrt(cnk) * 1.0001;
      const double e1 = 2.0 * (2.0 * dg * vn * ck + du * (cnk + fabs(y1) * (1.0 + delta) + eta)) * (1.0 + 1e-6);
      const bool biased = nk != nullptr;
      if (!(a2 < __builtin_inff()) || others_lower_bound(x2, vn, dg, du, biased) > x1 + e1) {
        label = k1;
      } else if ((unsigned)k2 < (unsigned)K &&
                 (!(a3 < __builtin_inff()) || others_lower_bound(x3, vn, dg, du, biased) > x1 + e1)) {
        // the exact argmin is k1 or k2: their exact distances (the re-rank's arithmetic)
        const uint16_t* vr = Vh + (size_t)(t0 + tid) * D;
        auto exact = [&](int k, double& dk, double& lk) {
          const uint16_t* cr = Ch + (size_t)k * D;
          dpair sum{0.0, 0.0};
          for (int c8 = 0; c8 < D; c8 += 8) {
            const uint4 va = *reinterpret_cast<const uint4*>(vr + c8), ca = *reinterpret_cast<const uint4*>(cr + c8);
            const uint32_t wv[4] = {va.x, va.y, va.z, va.w}, wc[4] = {ca.x, ca.y, ca.z, ca.w};
            for (int e = 0; e < 4; e++) {
              const double dl = (double)__uint_as_float(wv[e] << 16) - (double)__uint_as_float(wc[e] << 16);
              const double dh = (double)__uint_as_float(wv[e] & 0xffff0000u) - (double)__uint_as_float(wc[e] & 0xffff0000u);
              dp_add_sq(sum, dl);
              dp_add_sq(sum, dh);
            }
          }
          const dpair r = with_bias(dp_norm(sum), k);
          dk = r.hi; lk = r.lo;
        };
        // binary64 first: the terms are non-negative, so each computed distance (with b_k: one
        // more rounding) is within (D + 2) 2^-53 of its exact value, relatively; when the two
        // differ by more than both bounds their order is the exact one, otherwise the exact
        // pairs decide
        const uint16_t *ca = Ch + (size_t)k1 * D, *cb = Ch + (size_t)k2 * D;
        double sA = 0.0, sB = 0.0;
        for (int c8 = 0; c8 < D; c8 += 8) {
          const uint4 va = *reinterpret_cast<const uint4*>(vr + c8), xa = *reinterpret_cast<const uint4*>(ca + c8),
                      xb = *reinterpret_cast<const uint4*>(cb + c8);
          const uint32_t wv[4] = {va.x, va.y, va.z, va.w}, wa[4] = {xa.x, xa.y, xa.z, xa.w},
                         wb[4] = {xb.x, xb.y, xb.z, xb.w};
          for (int e = 0; e < 4; e++) {
            const double vl = (double)__uint_as_float(wv[e] << 16), vh = (double)__uint_as_float(wv[e] & 0xffff0000u);
            const double al = vl - (double)__uint_as_float(wa[e] << 16);
            const double ah = vh - (double)__uint_as_float(wa[e] & 0xffff0000u);
            const double bl = vl - (double)__uint_as_float(wb[e] << 16);
            const double bh = vh - (double)__uint_as_float(wb[e] & 0xffff0000u);
            sA = fma(al, al, sA);
            sA = fma(ah, ah, sA);
            sB = fma(bl, bl, sB);
            sB = fma(bh, bh, sB);
          }
        }
        if (nkh) {
          sA += (double)(lam * (float)nkh[k1]);
          sB += (double)(lam * (float)nkh[k2]);
        }
        if (fabs(sA - sB) > (D + 4) * 0x1p-52 * fmax(sA, sB)) {
          label = sB < sA ? k2 : k1;
        } else {
          double dA, lA, dB, lB;
          exact(k1, dA, lA);
          exact(k2, dB, lB);
          label = better(dB, lB, k2, dA, lA, k1) ? k2 : k1;
        }
      }
    }
    if (label >= 0) labels[(size_t)bh * N + t0 + tid] = label;
    else unsure[atomicAdd(&n_unsure, 1)] = tid;
  }
  __syncthreads();
  // exact re-rank of the uncertain tokens, in batches of RB tokens with two
  // barriers per batch: for each token the eight lanes of a lane group share one centroid
  // row (D/8 features each, so a row is one coalesced read) and the work-group's 32 lane
  // groups take centroids k = 32j + 8 wave + group. The partial sums are combined across the
  // lane group, the groups' winners across the wave, and the four waves' winners through LDS.
  // The squared bf16 differences are summed as exact binary64 pairs (TwoProduct, TwoSum),
  // so their order does not change them; a distance (with size penalties: plus b_k) is the
  // normalised pair (hi, lo), hi the nearest binary64 of the exact value and lo the exact
  // rest, ranked lexicographically (rounding is monotone); ties go to the lowest index.
  const int nu = n_unsure;
  constexpr int SL = D / 8;  // features per lane
  const int sub = lane & 7, grp = lane >> 3;
  auto load_slice = [&](const uint16_t* p, double* f) {
    for (int q = 0; q < SL / 8; q++) {
      const uint4 raw = *reinterpret_cast<const uint4*>(p + 8 * q);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      for (int e = 0; e < 4; e++) {
        f[8 * q + 2 * e] = (double)__uint_as_float(w[e] << 16);
        f[8 * q + 2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
      }
    }
  };
  for (int u0 = 0; u0 < nu; u0 += RB) {
    const int nb = min(RB, nu - u0);
    for (int j = 0; j < nb; j++) {
      const int t = t0 + unsure[u0 + j];
      double vf[SL];
      load_slice(Vh + (size_t)t * D + sub * SL, vf);
      double best = __builtin_inf(), blo = 0.0;
      int bk = 0x7fffffff;
      for (int kk = 0; kk < K; kk += 32) {
        const int k = kk + 8 * wave + grp;
        dpair s{0.0, 0.0};
        if (k < K) {
          double cf[SL];
          load_slice(Ch + (size_t)k * D + sub * SL, cf);
          for (int c = 0; c < SL; c++) dp_add_sq(s, vf[c] - cf[c]);
        }
        // butterfly over the lane group: every lane of it ends with the same exact pair
        dp_merge(s, dp_shfl_xor(s, 1));
        dp_merge(s, dp_shfl_xor(s, 2));
        dp_merge(s, dp_shfl_xor(s, 4));
        if (k < K) {
          const dpair r = with_bias(dp_norm(s), k);
          if (r.hi < best || (r.hi == best && r.lo < blo)) { best = r.hi; blo = r.lo; bk = k; }
        }
      }
      for (int o = 8; o < 64; o <<= 1) {
        const double d2 = __shfl_xor(best, o), l2 = __shfl_xor(blo, o);
        const int k2 = __shfl_xor(bk, o);
        if (better(d2, l2, k2, best, blo, bk)) { best = d2; blo = l2; bk = k2; }
      }
      if (lane == 0) rr[j][wave] = Exact{best, blo, bk};
    }
    __syncthreads();
    if (tid < nb) {
      Exact a = rr[tid][0];
      for (int w = 1; w < 4; w++) {
        const Exact& o = rr[tid][w];
        if (better(o.d, o.lo, o.k, a.d, a.lo, a.k)) a = o;
      }
      labels[(size_t)bh * N + t0 + unsure[u0 + tid]] = ((unsigned)a.k < (unsigned)K) ? a.k : 0;
    }
    __syncthreads();
  }
}

// Per-chunk label counts, counts[bh][chunk][k]: each work-group writes its K counts as one
// contiguous row.
__global__ __launch_bounds__(256) void cl_hist(const int32_t* __restrict__ labels, int N, int K, int nch,
                                               int32_t* __restrict__ counts) {
  extern __shared__ int hist[];
  const int ch = blockIdx.x, bh = blockIdx.y;
  for (int k = threadIdx.x; k < K; k += 256) hist[k] = 0;
  __syncthreads();
  const int t = ch * kChunk + threadIdx.x;
  if (t < N) {
    const int z = labels[(size_t)bh * N + t];
    atomicAdd(&hist[((unsigned)z < (unsigned)K) ? z : 0], 1);
  }
  __syncthreads();
  int32_t* row = counts + ((size_t)bh * nch + ch) * K;
  for (int k = threadIdx.x; k < K; k += 256) row[k] = hist[k];
}

// Stable counting sort, scan part 1: offsets[bh][chunk][k] = number of tokens labelled k in
// the chunks before `chunk` (chunk order), total[bh][k] = all of them. Work-group = 64
// clusters (lane = cluster) x 16 waves; wave w takes a contiguous range of chunks, so every
// access is a 256-byte row segment. Two passes over the wave's range: its sum, then (after
// an exclusive scan of the 16 sums through LDS) the running offsets.
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(64 * kScanWaves) void cl_scan_k(const int32_t* __restrict__ counts, int K, int nch,
                                                            int32_t* __restrict__ offsets, int32_t* __restrict__ total) {
  __shared__ int part[kScanWaves][64];
  const int bh = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + lane;
  const bool on = k < K;
  const int per = (nch + kScanWaves - 1) / kScanWaves;
  const int a = min(nch, w * per), b = min(nch, a + per);
  const int32_t* cnt = counts + (size_t)bh * nch * K + k;
  int32_t* off = offsets + (size_t)bh * nch * K + k;
  int s = 0;
  if (on)
    for (int c = a; c < b; c++) s += cnt[(size_t)c * K];
  part[w][lane] = s;
  __syncthreads();
  int run = 0;
  for (int v = 0; v < w; v++) run += part[v][lane];
  if (on) {
    for (int c = a; c < b; c++) {
      off[(size_t)c * K] = run;
      run += cnt[(size_t)c * K];
    }
    if (w == kScanWaves - 1) total[(size_t)bh * K + k] = run;
  }
}

// Scan part 2: cluster starts = exclusive scan of the totals (k order), sizes = totals.
__global__ __launch_bounds__(1024) void cl_scan_c(const int32_t* __restrict__ total, int K, int32_t* __restrict__ cstart,
                                                  int32_t* __restrict__ csize) {
  __shared__ int part[1024];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int per = (K + 1023) / 1024;
  const int a = min(K, tid * per), b = min(K, a + per);
  const int32_t* tt = total + (size_t)bh * K;
  int s = 0;
  for (int i = a; i < b; i++) s += tt[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = (tid >= o) ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int i = a; i < b; i++) {
    cstart[(size_t)bh * K + i] = run;
    csize[(size_t)bh * K + i] = tt[i];
    run += tt[i];
  }
}

__global__ __launch_bounds__(256) void cl_scatter(const int32_t* __restrict__ labels, int N, int K, int nch,
                                                  const int32_t* __restrict__ offsets, const int32_t* __restrict__ cstart,
                                                  int32_t* __restrict__ perm) {
  __shared__ int lab[kChunk];
  const int ch = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int t = ch * kChunk + tid;
  int z0 = (t < N) ? labels[(size_t)bh * N + t] : -1;
  if (t < N && (unsigned)z0 >= (unsigned)K) z0 = 0;
  lab[tid] = z0;
  __syncthreads();
  if (t < N) {
    const int z = lab[tid];
    int rank = 0;
    for (int i = 0; i < tid; i++) rank += (lab[i] == z);
    perm[(size_t)bh * N + cstart[(size_t)bh * K + z] + offsets[((size_t)bh * nch + ch) * K + z] + rank] = t;
  }
}

// C_k = fl32(exact mean of the member rows). 128 threads: the D channels in 16-byte
// chunks (D/8 threads per row) times 128*8/D row groups that take every G-th member; the
// exact partial sums (binary64 pairs) are combined across the row groups of a wave with lane
// shuffles and across the two waves in LDS (order-independent).
template <int D>
__device__ __forceinline__ void member_sums(const uint16_t* __restrict__ Vh, const int32_t* __restrict__ ph, int N,
                                            int n, dpair (*part)[D]) {
  constexpr int CH = D / 8, G = 128 / CH;
  const int chunk = threadIdx.x % CH, g = threadIdx.x / CH;
  dpair acc[8];
  for (int e = 0; e < 8; e++) acc[e] = dpair{0.0, 0.0};
  auto add_row = [&](const uint4 raw) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    for (int e = 0; e < 4; e++) {
      dp_add(acc[2 * e], (double)__uint_as_float(w[e] << 16));
      dp_add(acc[2 * e + 1], (double)__uint_as_float(w[e] & 0xffff0000u));
    }
  };
  auto load_row = [&](int i) {
    int row = ph[i];
    row = ((unsigned)row < (unsigned)N) ? row : 0;
    return *reinterpret_cast<const uint4*>(Vh + (size_t)row * D + 8 * chunk);
  };
  // four member rows in flight per row group (the index and row loads of one member are
  // dependent; members are independent); the sums are exact, so the order in which members
  // are added does not change the result
  int i = g;
  for (; i + 3 * G < n; i += 4 * G) {
    const uint4 r0 = load_row(i), r1 = load_row(i + G), r2 = load_row(i + 2 * G), r3 = load_row(i + 3 * G);
    add_row(r0); add_row(r1); add_row(r2); add_row(r3);
  }
  for (; i < n; i += G) add_row(load_row(i));
  for (int e = 0; e < 8; e++) {
    for (int o = CH; o < 64; o <<= 1) dp_merge(acc[e], dp_shfl_xor(acc[e], o));
    if ((threadIdx.x & 63) < CH) part[threadIdx.x >> 6][8 * chunk + e] = acc[e];
  }
}

// at least seven waves per SIMD (72 VGPRs): the pair sums keep more live values than the loads
// need, and the extra waves hide the dependent index and row loads (measured against five and six)
template <int D>
__global__ __launch_bounds__(128, 7) void cl_update(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ cstart, const int32_t* __restrict__ csize,
                                                 int N, int K, float* __restrict__ C) {
  __shared__ dpair part[2][D];
  const int k = blockIdx.x, bh = blockIdx.y;
  const int n = csize[(size_t)bh * K + k];
  if (n == 0) return;  // empty cluster keeps its centroid
  const int s0 = cstart[(size_t)bh * K + k];
  member_sums<D>(V + (size_t)bh * N * D, perm + (size_t)bh * N + s0, N, n, part);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 128) {
    dpair s = part[0][c];
    dp_merge(s, part[1][c]);
    C[((size_t)bh * K + k) * D + c] = dp_div_to_f32(s, (double)n);
  }
}

// k-means objective of the values under fixed labels and centroids (a drift statistic:
// the paper page's weakness list suggests detecting layout drift to refresh the
// clustering early). Partial sums of ||V_t - bf16(C_{z_t})||^2 over kCostTokens tokens per
// work-group: the difference of two bf16 values is exact in binary64, its square and the
// sums are binary64 roundings (relative error ~1e-13 over a head).
// Cross-step incremental update (the paper page's weakness list: centroids updated
// incrementally across denoising steps). Cluster k keeps a decayed member mass M_k; with A =
// decay * M_k (binary64, exact) and S_k = fl64(exact member sum), C_k = nearest binary32 of
// (A * C_k + S_k) / (A + n_k) with the product, the sum and the denominator rounded in
// binary64 op by op, and M_k = fl32(A + n_k). An empty cluster keeps C_k, M_k = fl32(A).
// six waves per SIMD (74 VGPRs): seven would spill
template <int D>
__global__ __launch_bounds__(128, 6) void cl_update_inc(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ cstart,
                                                     const int32_t* __restrict__ csize, int N, int K, float decay,
                                                     float* __restrict__ C, float* __restrict__ M) {
  __shared__ dpair part[2][D];
  const int k = blockIdx.x, bh = blockIdx.y;
  const size_t ck = (size_t)bh * K + k;
  const int n = csize[ck];
  const double A = (double)decay * (double)M[ck];
  if (n == 0) {
    if (threadIdx.x == 0) M[ck] = (float)A;
    return;
  }
  member_sums<D>(V + (size_t)bh * N * D, perm + (size_t)bh * N + cstart[ck], N, n, part);
  __syncthreads();  // every thread has read M[ck] before thread 0 writes it below
  const double den = A + (double)n;
  for (int c = threadIdx.x; c < D; c += 128) {
    dpair s = part[0][c];
    dp_merge(s, part[1][c]);
    const double num = A * (double)C[ck * D + c] + dp_norm(s).hi;
    C[ck * D + c] = div_to_f32(num, den);
  }
  if (threadIdx.x == 0) M[ck] = (float)den;
}

constexpr int kCostTokens = 1024;

template <int D>
__global__ __launch_bounds__(256) void cl_cost_part(const uint16_t* __restrict__ V, const float* __restrict__ C,
                                                    const int32_t* __restrict__ labels, int N, int K, int nblk,
                                                    double* __restrict__ part) {
  constexpr int CH = D / 8, G = 256 / CH;
  __shared__ double red[256];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int chunk = threadIdx.x % CH, g = threadIdx.x / CH;
  const int t0 = blk * kCostTokens, t1 = min(N, t0 + kCostTokens);
  double acc = 0.0;
  for (int t = t0 + g; t < t1; t += G) {
    int z = labels[(size_t)bh * N + t];
    z = ((unsigned)z < (unsigned)K) ? z : 0;
    const uint4 raw = *reinterpret_cast<const uint4*>(V + ((size_t)bh * N + t) * D + 8 * chunk);
    const float4 c0 = *reinterpret_cast<const float4*>(C + ((size_t)bh * K + z) * D + 8 * chunk);
    const float4 c1 = *reinterpret_cast<const float4*>(C + ((size_t)bh * K + z) * D + 8 * chunk + 4);
    const float cf[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    for (int e = 0; e < 8; e++) {
      const float v = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
      const double df = (double)v - (double)bf16_to_f32(f32_to_bf16(cf[e]));
      acc += df * df;
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(size_t)bh * nblk + blk] = red[0];
}

__global__ void cl_cost_final(const double* __restrict__ part, int nblk, int N, int BH, double* __restrict__ cost) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  double s = 0.0;
  for (int b = 0; b < nblk; b++) s += part[(size_t)bh * nblk + b];
  cost[bh] = s / (double)N;
}

}  // namespace vc

using namespace vc;

extern "C" size_t vc_cluster_cost_ws_bytes(int B, int H, int N) {
  return (size_t)B * H * ((N + kCostTokens - 1) / kCostTokens) * sizeof(double) + 256;
}

extern "C" int vc_launch_cluster_cost(const void* V, const float* C, const int32_t* labels, int B, int H, int N, int d,
                                      int K, double* cost, void* ws, hipStream_t st) {
  const int BH = B * H, nblk = (N + kCostTokens - 1) / kCostTokens;
  double* part = (double*)ws;
  if (d == 128) cl_cost_part<128><<<dim3(nblk, BH), 256, 0, st>>>((const uint16_t*)V, C, labels, N, K, nblk, part);
  else cl_cost_part<64><<<dim3(nblk, BH), 256, 0, st>>>((const uint16_t*)V, C, labels, N, K, nblk, part);
  cl_cost_final<<<(BH + 63) / 64, 64, 0, st>>>(part, nblk, N, BH, cost);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" size_t vc_cluster_ws_bytes(int B, int H, int N, int d, int K) {
  const size_t BH = (size_t)B * H, nch = ((size_t)N + kChunk - 1) / kChunk;
  return BH * K * d * sizeof(float) + BH * K * sizeof(float) + 2 * BH * K * nch * sizeof(int32_t) +
         3 * BH * K * sizeof(int32_t) + 1024;
}

__global__ void cl_copy_sizes(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// nk_io == nullptr: plain Lloyd iterations (lam unused). Otherwise size-penalised: the first
// assignment uses the sizes in nk_io, later ones the sizes of the previous assignment, and
// nk_io receives the sizes of the last one.
extern "C" int vc_launch_cluster(const void* Vv, int B, int H, int N, int d, int K, int iters, int cold, float* C,
                                 int32_t* labels, int32_t* perm, void* ws, hipStream_t st, float lam,
                                 int32_t* nk_io) {
  const uint16_t* V = (const uint16_t*)Vv;
  const int BH = B * H, nch = (N + kChunk - 1) / kChunk;
  char* w = (char*)ws;
  uint16_t* chat = (uint16_t*)w; w += (size_t)BH * K * d * sizeof(float);
  float* cnorm = (float*)w; w += (size_t)BH * K * sizeof(float);
  int32_t* counts = (int32_t*)w; w += (size_t)BH * K * nch * sizeof(int32_t);
  int32_t* offs = (int32_t*)w; w += (size_t)BH * K * nch * sizeof(int32_t);
  int32_t* cstart = (int32_t*)w; w += (size_t)BH * K * sizeof(int32_t);
  int32_t* csize = (int32_t*)w; w += (size_t)BH * K * sizeof(int32_t);
  int32_t* ctotal = (int32_t*)w;
  if (cold) cl_cold<<<dim3(K, BH), d, 0, st>>>(V, C, N, K, d);
  const dim3 gmf((N + kAssignTokens - 1) / kAssignTokens, BH), gch(nch, BH), gk(K, BH);
  for (int it = 0; it < iters; it++) {
    const int32_t* nk = nk_io ? (it == 0 ? nk_io : csize) : nullptr;
    cl_prep<<<gk, d, 0, st>>>(C, chat, cnorm, K, d, nk, lam);
    if (d == 128) cl_assign_mfma<128><<<gmf, 256, 0, st>>>(V, chat, cnorm, N, K, labels, nk, lam);
    else cl_assign_mfma<64><<<gmf, 256, 0, st>>>(V, chat, cnorm, N, K, labels, nk, lam);
    cl_hist<<<gch, 256, K * sizeof(int), st>>>(labels, N, K, nch, counts);
    cl_scan_k<<<dim3((K + 63) / 64, BH), 64 * kScanWaves, 0, st>>>(counts, K, nch, offs, ctotal);
    cl_scan_c<<<BH, 1024, 0, st>>>(ctotal, K, cstart, csize);
    cl_scatter<<<gch, 256, 0, st>>>(labels, N, K, nch, offs, cstart, perm);
    if (d == 128) cl_update<128><<<gk, 128, 0, st>>>(V, perm, cstart, csize, N, K, C);
    else cl_update<64><<<gk, 128, 0, st>>>(V, perm, cstart, csize, N, K, C);
  }
  if (nk_io && iters > 0) cl_copy_sizes<<<(BH * K + 255) / 256, 256, 0, st>>>(csize, nk_io, BH * K);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// One incremental step: optional assignment to bf16(C) (plain, no size penalty), the stable
// counting sort of the labels, then the decayed update. Labels outside [0, K) read as 0.
extern "C" int vc_launch_cluster_inc(const void* Vv, int B, int H, int N, int d, int K, float decay, int assign,
                                     float* C, float* M, int32_t* labels, int32_t* perm, void* ws, hipStream_t st) {
  const uint16_t* V = (const uint16_t*)Vv;
  const int BH = B * H, nch = (N + kChunk - 1) / kChunk;
  char* w = (char*)ws;
  uint16_t* chat = (uint16_t*)w; w += (size_t)BH * K * d * sizeof(float);
  float* cnorm = (float*)w; w += (size_t)BH * K * sizeof(float);
  int32_t* counts = (int32_t*)w; w += (size_t)BH * K * nch * sizeof(int32_t);
  int32_t* offs = (int32_t*)w; w += (size_t)BH * K * nch * sizeof(int32_t);
  int32_t* cstart = (int32_t*)w; w += (size_t)BH * K * sizeof(int32_t);
  int32_t* csize = (int32_t*)w; w += (size_t)BH * K * sizeof(int32_t);
  int32_t* ctotal = (int32_t*)w;
  const dim3 gmf((N + kAssignTokens - 1) / kAssignTokens, BH), gch(nch, BH), gk(K, BH);
  if (assign) {
    cl_prep<<<gk, d, 0, st>>>(C, chat, cnorm, K, d, nullptr, 0.0f);
    if (d == 128) cl_assign_mfma<128><<<gmf, 256, 0, st>>>(V, chat, cnorm, N, K, labels, nullptr, 0.0f);
    else cl_assign_mfma<64><<<gmf, 256, 0, st>>>(V, chat, cnorm, N, K, labels, nullptr, 0.0f);
  }
  cl_hist<<<gch, 256, K * sizeof(int), st>>>(labels, N, K, nch, counts);
  cl_scan_k<<<dim3((K + 63) / 64, BH), 64 * kScanWaves, 0, st>>>(counts, K, nch, offs, ctotal);
  cl_scan_c<<<BH, 1024, 0, st>>>(ctotal, K, cstart, csize);
  cl_scatter<<<gch, 256, 0, st>>>(labels, N, K, nch, offs, cstart, perm);
  if (d == 128) cl_update_inc<128><<<gk, 128, 0, st>>>(V, perm, cstart, csize, N, K, decay, C, M);
  else cl_update_inc<64><<<gk, 128, 0, st>>>(V, perm, cstart, csize, N, K, decay, C, M);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int vc_max_clusters(void) { return kMaxClusters; }

// ---------------------------------------------------------------------------
// Exponent range of a tensor per (b,h), the quantity the exactness conditions of the exact
// (binary64-pair) sums and distances are stated in: over the nonzero finite elements, the largest exponent
// e = floor(log2|x|) and the smallest exponent of a lowest set significand bit (every element
// is an integer multiple of 2^that). kind 0: bf16 bit patterns; 1: binary32; 2: binary32 taken
// as the bf16 value it rounds to (nearest even), as the assignment reads centroids.
namespace vc {

__global__ void span_init(int32_t* __restrict__ out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    out[2 * i] = INT32_MIN;
    out[2 * i + 1] = INT32_MAX;
  }
}

// e and q of one element given its biased exponent field, significand field and format widths;
// returns false for zero, infinity and NaN
__device__ __forceinline__ bool elem_exponents(uint32_t ef, uint32_t mant, int mbits, int& e, int& q) {
  const uint32_t emaxf = 0xFFu;
  if (ef == emaxf) return false;
  if (ef == 0 && mant == 0) return false;
  const int qsub = -126 - mbits;  // exponent of the last bit of a subnormal
  if (ef == 0) {
    e = (31 - __clz(mant)) + qsub;
    q = qsub + __ffs(mant) - 1;
  } else {
    const uint32_t sig = mant | (1u << mbits);
    e = (int)ef - 127;
    q = e - mbits + __ffs(sig) - 1;
  }
  return true;
}

__global__ __launch_bounds__(256) void span_kernel(const void* __restrict__ X, int kind, long long per_head,
                                                   int32_t* __restrict__ out) {
  __shared__ int red[2][4];
  const int bh = blockIdx.y;
  int emax = INT32_MIN, qmin = INT32_MAX;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < per_head; i += stride) {
    uint32_t ef, mant;
    int mbits;
    if (kind == 0) {
      const uint32_t h = reinterpret_cast<const uint16_t*>(X)[(size_t)bh * per_head + i];
      ef = (h >> 7) & 0xFFu; mant = h & 0x7Fu; mbits = 7;
    } else {
      uint32_t f = __float_as_uint(reinterpret_cast<const float*>(X)[(size_t)bh * per_head + i]);
      if (kind == 2) {
        if (((f >> 23) & 0xFFu) == 0xFFu) continue;  // infinity or NaN
        f = (uint32_t)f32_to_bf16(__uint_as_float(f)) << 16;
        ef = (f >> 23) & 0xFFu; mant = (f >> 16) & 0x7Fu; mbits = 7;
      } else {
        ef = (f >> 23) & 0xFFu; mant = f & 0x7FFFFFu; mbits = 23;
      }
    }
    int e, q;
    if (elem_exponents(ef, mant, mbits, e, q)) {
      emax = max(emax, e);
      qmin = min(qmin, q);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    emax = max(emax, __shfl_xor(emax, o));
    qmin = min(qmin, __shfl_xor(qmin, o));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = emax; red[1][w] = qmin; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; k++) { emax = max(emax, red[0][k]); qmin = min(qmin, red[1][k]); }
    if (emax != INT32_MIN) {  // max and min are order-free: the result is deterministic
      atomicMax(&out[2 * bh], emax);
      atomicMin(&out[2 * bh + 1], qmin);
    }
  }
}

}  // namespace vc

extern "C" int vc_launch_exponent_span(const void* X, int kind, int BH, long long per_head, int32_t* out,
                                       hipStream_t st) {
  vc::span_init<<<(BH + 255) / 256, 256, 0, st>>>(out, BH);
  const long long blocks = (per_head + 256LL * 16 - 1) / (256LL * 16);
  const int gx = (int)(blocks < 1024 ? (blocks < 1 ? 1 : blocks) : 1024);
  vc::span_kernel<<<dim3(gx, BH), 256, 0, st>>>(X, kind, per_head, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
