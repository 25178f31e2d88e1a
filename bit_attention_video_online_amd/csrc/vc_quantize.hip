// vc_quantize.hip -- fused quantiser of the VC-Attention hot path for gfx950.
//
// Paper page (paper.rainbus.top), method step (2), and study notes section 2-2:
// V' = V[pi] is cut into 128-row blocks, each block's mean mu_j is removed and only
// the residual R = V' - mu_j is quantised (per-channel E4M3), the mean kept in 16
// bits. Q and the smoothed, permuted keys get one E4M3 scale per 128-row block.
//
// Three launches (both global statistics -- the key channel mean and the residual
// channel maximum -- need a pass over all N tokens before codes can be written):
//   quant_stats  : per (b,h,block): Q codes + scale; V' block mean (bf16) and the
//                  block's residual |max| per channel; exact key channel partial sums.
//   quant_reduce : per (b,h): kbar = fl32(exact mean), sV = fl32(amax/448), 448/amax.
//   quant_apply  : per (b,h,block): K~' codes + scale; residual codes (block-transposed
//                  layout) and mu / sV.
// Optional preprocessing that the pages' fused quantiser also absorbs: RoPE on Q and K
// (interleaved channel pairs, caller's binary32 cos/sin tables [N, d/2], binary32
// products, result rounded to bf16) and the Q/K Hadamard rotation (unnormalised
// Sylvester matrix by the fast Walsh-Hadamard transform, ascending stages, binary32; its
// factor 1/d is folded exactly into sQ').
// Tiles stay in registers (no LDS staging): every load is a 16-byte vector of one token
// row (rows of V' and K' gathered through pi) and per-channel reductions use lane
// shuffles plus a small LDS step. The 128-term and N-term sums of bfloat16 values are
// carried as binary64 pairs (hi + lo, error-free additions), exact for wide exponent spans.
#include "vc_exact.h"

static_assert(vc::kBlock == 128, "block means are scaled by 2^-7");

namespace vc {

constexpr int kQThreads = 256;

// Thread layout of a 128 x D tile: 16-byte vectors (8 bf16). Thread t owns column chunk
// t % CH (channels 8*chunk .. +7) of the RPT consecutive rows RPT*(t / CH) .. +RPT-1, so a
// wave-wide load or store instruction covers whole rows (coalesced), and per-channel
// reductions run over the threads that share a chunk: lanes xor multiples of CH inside a
// wave, then the four waves through LDS.
template <int D>
struct Lay {
  static constexpr int CH = D / 8;                   // chunks per row
  static constexpr int RG = kQThreads / CH;          // row groups
  static constexpr int RPT = kBlock / RG;            // rows per thread (8 or 4)
};

__device__ __forceinline__ void unpack8(uint4 raw, float* x) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  for (int k = 0; k < 4; k++) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

// rows of a tile, gathered through `perm_blk` (or contiguous when NULL); an out-of-range
// permutation entry reads row 0 instead of out of bounds
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* base, const int32_t* perm_blk, int nrows, float (&x)[Lay<D>::RPT][8]) {
  constexpr int CH = Lay<D>::CH, RPT = Lay<D>::RPT;
  const int chunk = threadIdx.x % CH, rg = threadIdx.x / CH;
  for (int i = 0; i < RPT; i++) {
    const int r = RPT * rg + i;
    int src = perm_blk ? perm_blk[r] : r;
    src = ((unsigned)src < (unsigned)nrows) ? src : 0;
    unpack8(*reinterpret_cast<const uint4*>(base + (size_t)src * D + 8 * chunk), x[i]);
  }
}

constexpr uint32_t kFlagHadamard = 16u;  // flag bit of the Q/K rotation
constexpr uint32_t kFlagMxfp4 = 32u;     // flag bit of the 4-bit (MXFP4) value residual

// MXFP4 value residual. E2M1 code of x (|x| <= 6): nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6,
// ties to the even mantissa; a value that rounds to zero keeps a plus sign.
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return (c != 0u && x < 0.0f) ? (c | 8u) : c;
}
// group scale exponent: the smallest e with amax <= 6 * 2^e (0 for amax = 0), within [-127, 127]
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return 0;
  int e = ilogbf(amax) - 2;
  while (ldexpf(6.0f, e) < amax) e++;
  while (ldexpf(6.0f, e - 1) >= amax) e--;
  return min(127, max(-127, e));
}

// RoPE on the thread's RPT rows (channel pairs 4*chunk .. +3 of each row); `pos` gives the
// token whose angles apply (its row in the tables). Each rotated value is rounded to bf16.
template <int D>
__device__ __forceinline__ void rope_tile(float (&x)[Lay<D>::RPT][8], const float* __restrict__ rc,
                                          const float* __restrict__ rs, const int (&pos)[Lay<D>::RPT]) {
  constexpr int RPT = Lay<D>::RPT;
  const int chunk = threadIdx.x % Lay<D>::CH;
  for (int i = 0; i < RPT; i++) {
    const float4 c = *reinterpret_cast<const float4*>(rc + (size_t)pos[i] * (D / 2) + 4 * chunk);
    const float4 sn = *reinterpret_cast<const float4*>(rs + (size_t)pos[i] * (D / 2) + 4 * chunk);
    const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
    for (int k = 0; k < 4; k++) {
      const float a = x[i][2 * k], b = x[i][2 * k + 1];
      const float ac = a * cc[k], bsn = b * ss[k], asn = a * ss[k], bc = b * cc[k];
      x[i][2 * k] = bf16_to_f32(f32_to_bf16(ac - bsn));
      x[i][2 * k + 1] = bf16_to_f32(f32_to_bf16(asn + bc));
    }
  }
}

// Row positions of the thread's rows: contiguous block rows, or the permutation's sources
// (clamped like load_tile)
template <int D>
__device__ __forceinline__ void tile_rows(const int32_t* perm_blk, int row0, int nrows, int (&pos)[Lay<D>::RPT]) {
  constexpr int RPT = Lay<D>::RPT;
  const int rg = threadIdx.x / Lay<D>::CH;
  for (int i = 0; i < RPT; i++) {
    const int r = RPT * rg + i;
    int src = perm_blk ? perm_blk[r] : row0 + r;
    pos[i] = ((unsigned)src < (unsigned)nrows) ? src : 0;
  }
}

// Unnormalised fast Walsh-Hadamard transform of every row of the tile: stages h = 1, 2, 4
// inside the thread's 8 channels, then h = 8, 16, ... across the lanes that hold the other
// chunks of the row (chunk bit k = lane bit k); the pair (i, i+h) becomes (a+b, a-b).
template <int D>
__device__ __forceinline__ void fwht_tile(float (&x)[Lay<D>::RPT][8]) {
  constexpr int CH = Lay<D>::CH, RPT = Lay<D>::RPT;
  const int chunk = threadIdx.x % CH;
  for (int i = 0; i < RPT; i++)
    for (int h = 1; h < 8; h <<= 1)
      for (int e = 0; e < 8; e++)
        if (!(e & h)) {
          const float a = x[i][e], b = x[i][e + h];
          x[i][e] = a + b;
          x[i][e + h] = a - b;
        }
  for (int m = 1; m < CH; m <<= 1) {
    const bool upper = (chunk & m) != 0;
    for (int i = 0; i < RPT; i++)
      for (int e = 0; e < 8; e++) {
        const float p = __shfl_xor(x[i][e], m);
        x[i][e] = upper ? p - x[i][e] : x[i][e] + p;
      }
  }
}

// reductions over the threads that share a chunk (lane bits >= log2(CH), then waves)
template <int D>
__device__ __forceinline__ dpair chunk_sum_wave(dpair v) {
  for (int o = Lay<D>::CH; o < 64; o <<= 1) dp_merge(v, dp_shfl_xor(v, o));
  return v;
}
template <int D>
__device__ __forceinline__ float chunk_max_wave(float v) {
  for (int o = Lay<D>::CH; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// whole-block max over 256 threads
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// one scale for the tile: s = fl32(amax/448), codes e4m3(fl32(x * fl32(448/amax)));
// amax = 0 gives scale 1 and zero codes. Codes row-major, 8 bytes per row and thread.
template <int D>
__device__ __forceinline__ float quant_rows(float (&x)[Lay<D>::RPT][8], uint8_t* dst, float* red) {
  constexpr int CH = Lay<D>::CH, RPT = Lay<D>::RPT;
  const int chunk = threadIdx.x % CH, rg = threadIdx.x / CH;
  float a = 0.0f;
  for (int i = 0; i < RPT; i++)
    for (int e = 0; e < 8; e++) a = fmaxf(a, fabsf(x[i][e]));
  a = block_max(a, red);
  float s, inv;
  if (a > 0.0f) { s = a / 448.0f; inv = 448.0f / a; } else { s = 1.0f; inv = 0.0f; }
  for (int i = 0; i < RPT; i++) {
    const uint32_t lo = e4m3x4_from_f32(x[i][0] * inv, x[i][1] * inv, x[i][2] * inv, x[i][3] * inv);
    const uint32_t hi = e4m3x4_from_f32(x[i][4] * inv, x[i][5] * inv, x[i][6] * inv, x[i][7] * inv);
    *reinterpret_cast<uint2*>(dst + (size_t)(RPT * rg + i) * D + 8 * chunk) = make_uint2(lo, hi);
  }
  return s;
}

// per-channel exact column sums of the tile as binary64 pairs (exact, so the summation
// order is immaterial); result for channel c in colsum[c] (LDS), valid after the call
template <int D>
__device__ __forceinline__ void column_sums(const float (&x)[Lay<D>::RPT][8], dpair* part, dpair* colsum) {
  constexpr int CH = Lay<D>::CH, RPT = Lay<D>::RPT;
  const int chunk = threadIdx.x % CH, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = 0; e < 8; e++) {
    dpair acc{0.0, 0.0};
    for (int i = 0; i < RPT; i++) dp_add(acc, (double)x[i][e]);
    acc = chunk_sum_wave<D>(acc);
    if (lane < CH) part[w * D + 8 * chunk + e] = acc;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    dpair a = part[threadIdx.x];
    for (int q = 1; q < 4; q++) dp_merge(a, part[q * D + threadIdx.x]);
    colsum[threadIdx.x] = a;
  }
  __syncthreads();
}

// ROPE / HAD select the optional preprocessing at compile time, so the plain path keeps
// its small register footprint.
template <int D, bool ROPE, bool HAD>
__global__ __launch_bounds__(kQThreads) void quant_stats(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                         const float* __restrict__ rc, const float* __restrict__ rs,
                                                         int N, uint32_t flags, float cL,
                                                         uint8_t* __restrict__ Qq, float* __restrict__ sQ,
                                                         uint16_t* __restrict__ mu, dpair* __restrict__ ksum,
                                                         float* __restrict__ vamax) {
  constexpr int CH = Lay<D>::CH, RPT = Lay<D>::RPT;
  __shared__ float red[4];
  __shared__ dpair part[4 * D];
  __shared__ dpair colsum[D];
  __shared__ float pmax[4 * D];
  const int nb = N / kBlock;
  const int j = blockIdx.x, bh = blockIdx.y;
  const size_t head = (size_t)bh * N * D, jrow = (size_t)j * kBlock * D;
  const int32_t* pblk = perm ? perm + (size_t)bh * N + (size_t)j * kBlock : nullptr;
  const int chunk = threadIdx.x % CH, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float x[RPT][8];

  int pos[RPT];
  if (ROPE) tile_rows<D>(nullptr, j * kBlock, N, pos);

  // ---- Q block (original order): codes and scale
  load_tile<D>(Q + head + jrow, nullptr, kBlock, x);
  if (ROPE) rope_tile<D>(x, rc, rs, pos);
  if (HAD) fwht_tile<D>(x);
  const float s = quant_rows<D>(x, Qq + head + jrow, red);
  if (threadIdx.x == 0) sQ[(size_t)bh * nb + j] = HAD ? ldexpf(s * cL, -__builtin_ctz(D)) : s * cL;

  // ---- key channel partial sums (token order is irrelevant for a sum)
  if (flags & 1u) {
    load_tile<D>(K + head + jrow, nullptr, kBlock, x);
    if (ROPE) rope_tile<D>(x, rc, rs, pos);
    column_sums<D>(x, part, colsum);
    if (threadIdx.x < D) ksum[((size_t)bh * nb + j) * D + threadIdx.x] = colsum[threadIdx.x];
  }

  // ---- V' block: mean mu = bf16(exact mean) and the residual channel maximum
  if (pblk) load_tile<D>(V + head, pblk, N, x);
  else load_tile<D>(V + head + jrow, nullptr, kBlock, x);
  float m[8];
  if (flags & 2u) {
    column_sums<D>(x, part, colsum);
    for (int e = 0; e < 8; e++) m[e] = bf16_to_f32(dp_to_bf16_scaled(colsum[8 * chunk + e], -7));  // / kBlock
    if (threadIdx.x < D) mu[((size_t)bh * nb + j) * D + threadIdx.x] = dp_to_bf16_scaled(colsum[threadIdx.x], -7);
  } else {
    for (int e = 0; e < 8; e++) m[e] = 0.0f;
    if (mu != nullptr && threadIdx.x < D) mu[((size_t)bh * nb + j) * D + threadIdx.x] = 0;
  }
  for (int e = 0; e < 8; e++) {
    float a = 0.0f;
    for (int i = 0; i < RPT; i++) a = fmaxf(a, fabsf(x[i][e] - m[e]));
    a = chunk_max_wave<D>(a);
    if (lane < CH) pmax[w * D + 8 * chunk + e] = a;
  }
  __syncthreads();
  if (threadIdx.x < D)
    vamax[((size_t)bh * nb + j) * D + threadIdx.x] =
        fmaxf(fmaxf(pmax[threadIdx.x], pmax[D + threadIdx.x]), fmaxf(pmax[2 * D + threadIdx.x], pmax[3 * D + threadIdx.x]));
}

// Per (b,h): kbar = fl32(exact mean) of the keys, residual scale sV = fl32(amax/448) and
// 448/amax. Work-group (bh, channel slice of 16): channel c = slice*16 + t % 16, group
// t / 16 takes every 16th block (two chains); the exact sums make the order immaterial.
constexpr int kRedCh = 16;
template <int D>
__global__ __launch_bounds__(kQThreads) void quant_reduce(int N, uint32_t flags, const dpair* __restrict__ ksum,
                                                          const float* __restrict__ vamax, float* __restrict__ kbar,
                                                          float* __restrict__ sV, float* __restrict__ vinv) {
  constexpr int G = kQThreads / kRedCh;
  __shared__ dpair ps[kQThreads];
  __shared__ float pm[kQThreads];
  const int nb = N / kBlock;
  const int bh = blockIdx.x, c = blockIdx.y * kRedCh + threadIdx.x % kRedCh, g = threadIdx.x / kRedCh;
  dpair t0{0.0, 0.0}, t1{0.0, 0.0};
  float a0 = 0.0f, a1 = 0.0f;
  int jb = g;
  for (; jb + G < nb; jb += 2 * G) {  // two independent chains per thread
    if (flags & 1u) {
      dp_merge(t0, ksum[((size_t)bh * nb + jb) * D + c]);
      dp_merge(t1, ksum[((size_t)bh * nb + jb + G) * D + c]);
    }
    a0 = fmaxf(a0, vamax[((size_t)bh * nb + jb) * D + c]);
    a1 = fmaxf(a1, vamax[((size_t)bh * nb + jb + G) * D + c]);
  }
  if (jb < nb) {
    if (flags & 1u) dp_merge(t0, ksum[((size_t)bh * nb + jb) * D + c]);
    a0 = fmaxf(a0, vamax[((size_t)bh * nb + jb) * D + c]);
  }
  dp_merge(t0, t1);
  ps[threadIdx.x] = t0;
  pm[threadIdx.x] = fmaxf(a0, a1);
  __syncthreads();
  if (g == 0) {
    dpair t{0.0, 0.0};
    float a = 0.0f;
    for (int k = 0; k < G; k++) { dp_merge(t, ps[k * kRedCh + threadIdx.x]); a = fmaxf(a, pm[k * kRedCh + threadIdx.x]); }
    kbar[(size_t)bh * D + c] = (flags & 1u) ? dp_div_to_f32(t, (double)N) : 0.0f;
    float s, inv;
    if (flags & kFlagMxfp4) { s = 1.0f; inv = 0.0f; }  // the group scales carry the range
    else if (a > 0.0f) { s = a / 448.0f; inv = 448.0f / a; } else { s = 1.0f; inv = 0.0f; }
    sV[(size_t)bh * D + c] = s;
    vinv[(size_t)bh * D + c] = inv;
  }
}

template <int D, bool ROPE, bool HAD, bool MX>
__global__ __launch_bounds__(kQThreads) void quant_apply(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                         const int32_t* __restrict__ perm, const float* __restrict__ rc,
                                                         const float* __restrict__ rs, int N, uint32_t flags,
                                                         const float* __restrict__ kbar, const float* __restrict__ sV,
                                                         const float* __restrict__ vinv, const uint16_t* __restrict__ mu,
                                                         uint8_t* __restrict__ Kq, float* __restrict__ sK,
                                                         uint8_t* __restrict__ Vq, float* __restrict__ mu_scaled,
                                                         uint16_t* __restrict__ mu_pack) {
  constexpr int CH = Lay<D>::CH, RPT = Lay<D>::RPT;
  __shared__ float red[4];
  const int nb = N / kBlock;
  const int j = blockIdx.x, bh = blockIdx.y;
  const size_t head = (size_t)bh * N * D, jrow = (size_t)j * kBlock * D;
  const int32_t* pblk = perm ? perm + (size_t)bh * N + (size_t)j * kBlock : nullptr;
  const int chunk = threadIdx.x % CH, rg = threadIdx.x / CH;
  float x[RPT][8];

  // ---- K~' = fl32(K[pi] - kbar), one scale per block, row-major codes
  {
    const float4 k0 = *reinterpret_cast<const float4*>(kbar + (size_t)bh * D + 8 * chunk);
    const float4 k1 = *reinterpret_cast<const float4*>(kbar + (size_t)bh * D + 8 * chunk + 4);
    const float kb[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    if (pblk) load_tile<D>(K + head, pblk, N, x);
    else load_tile<D>(K + head + jrow, nullptr, kBlock, x);
    if (ROPE) {  // the angles of each key's original position
      int pos[RPT];
      tile_rows<D>(pblk, j * kBlock, N, pos);
      rope_tile<D>(x, rc, rs, pos);
    }
    for (int i = 0; i < RPT; i++)
      for (int e = 0; e < 8; e++) x[i][e] = x[i][e] - kb[e];
    if (HAD) fwht_tile<D>(x);
    const float s = quant_rows<D>(x, Kq + head + jrow, red);
    if (threadIdx.x == 0) sK[(size_t)bh * nb + j] = s;
  }

  // ---- residual codes of V'[block j], block-transposed: Vq[c][t]; each thread stores the
  // RPT consecutive tokens of its 8 channels
  {
    const float4 v0 = *reinterpret_cast<const float4*>(vinv + (size_t)bh * D + 8 * chunk);
    const float4 v1 = *reinterpret_cast<const float4*>(vinv + (size_t)bh * D + 8 * chunk + 4);
    const float inv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float m[8];
    if (flags & 2u) unpack8(*reinterpret_cast<const uint4*>(mu + ((size_t)bh * nb + j) * D + 8 * chunk), m);
    else for (int e = 0; e < 8; e++) m[e] = 0.0f;
    if (pblk) load_tile<D>(V + head, pblk, N, x);
    else load_tile<D>(V + head + jrow, nullptr, kBlock, x);
    uint8_t* vb = Vq + head + jrow;
    if (MX) {
      // MXFP4: codes [c][64 bytes] then E8M0 scales [c][4] at byte 64 D of the block. Token t
      // of half q = t>>6 is nibble p = 16((t&63)>>5) + (t&15) of lane group g = (t>>4)&1, at
      // byte 32q + 16g + p/2 (low nibble first) -- the operand order of the block-scaled MFMA,
      // whose per-lane scale covers exactly group 2q + g of a channel.
      __shared__ uint32_t gmax[4 * D];
      for (int i = threadIdx.x; i < 4 * D; i += kQThreads) gmax[i] = 0u;
      __syncthreads();
      const int t0 = RPT * rg;
      const int q = t0 >> 6, g = (t0 >> 4) & 1, G = 2 * q + g;
      const int p0 = 16 * ((t0 & 63) >> 5) + (t0 & 15);
      for (int i = 0; i < RPT; i++)
        for (int e = 0; e < 8; e++) x[i][e] = x[i][e] - m[e];
      for (int e = 0; e < 8; e++) {
        float a = 0.0f;
        for (int i = 0; i < RPT; i++) a = fmaxf(a, fabsf(x[i][e]));
        atomicMax(&gmax[G * D + 8 * chunk + e], __float_as_uint(a));  // order-free for non-negative floats
      }
      __syncthreads();
      for (int e = 0; e < 8; e++) {
        const int ex = mx_exponent(__uint_as_float(gmax[G * D + 8 * chunk + e]));
        uint32_t wd = 0u;
        for (int i = 0; i < RPT; i++) wd |= e2m1_code(ldexpf(x[i][e], -ex)) << (4 * i);
        uint8_t* dst = vb + (size_t)(8 * chunk + e) * 64 + 32 * q + 16 * g + p0 / 2;
        if (RPT == 8) *reinterpret_cast<uint32_t*>(dst) = wd;
        else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)wd;
      }
      for (int idx = threadIdx.x; idx < 4 * D; idx += kQThreads)
        vb[64 * D + idx] = (uint8_t)(mx_exponent(__uint_as_float(gmax[(idx & 3) * D + (idx >> 2)])) + 127);
    } else
    for (int e = 0; e < 8; e++) {
      uint32_t wds[RPT / 4];
      for (int k = 0; k < RPT / 4; k++)
        wds[k] = e4m3x4_from_f32((x[4 * k + 0][e] - m[e]) * inv[e], (x[4 * k + 1][e] - m[e]) * inv[e],
                                 (x[4 * k + 2][e] - m[e]) * inv[e], (x[4 * k + 3][e] - m[e]) * inv[e]);
      uint8_t* dst = vb + (size_t)(8 * chunk + e) * kBlock + RPT * rg;
      if (RPT == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(wds[0], wds[RPT / 4 - 1]);
      else *reinterpret_cast<uint32_t*>(dst) = wds[0];
    }
  }

  // ---- mu / sV, and the packed mean operand of the attention kernel
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    const float sv = sV[(size_t)bh * D + c];
    const float m = (flags & 2u) ? bf16_to_f32(mu[((size_t)bh * nb + j) * D + c]) : 0.0f;
    if (mu_scaled) mu_scaled[((size_t)bh * nb + j) * D + c] = (flags & 2u) ? m / sv : 0.0f;
    // mean-restoration operand, laid out as the A operands of two v_mfma_f32_32x32x16_bf16
    // per 32-channel block: [chunk of 8 key blocks][d-block][MFMA t][lane][8]. MFMA 0:
    // lanes 0-31 and 32-63 hold bf16(ms); MFMA 1: lanes 0-31 bf16(ms - bf16(ms)), lanes
    // 32-63 zero; lane l carries channel 32*d-block + l%32, element s key block 8*chunk + s
    // (zero past the last key block). The last block of each chunk writes the whole chunk,
    // from the chunk's block means, as four 16-byte stores per channel.
    const int s8 = j % 8;
    if (mu_pack && (s8 == 7 || j == nb - 1)) {
      const int nc = (nb + 7) / 8, ch = j / 8, db = c / 32, r = c % 32;
      uint32_t hw[4] = {0u, 0u, 0u, 0u}, lw[4] = {0u, 0u, 0u, 0u};
      for (int t = 0; t <= s8; t++) {
        const float mt = (flags & 2u) ? bf16_to_f32(mu[((size_t)bh * nb + 8 * ch + t) * D + c]) : 0.0f;
        const float ms = (flags & 2u) ? mt / sv : 0.0f;
        const uint32_t hi = f32_to_bf16(ms);
        const uint32_t lo = f32_to_bf16(ms - bf16_to_f32((uint16_t)hi));
        hw[t / 2] |= hi << (16 * (t & 1));
        lw[t / 2] |= lo << (16 * (t & 1));
      }
      uint4* base = reinterpret_cast<uint4*>(mu_pack + ((((size_t)bh * nc + ch) * (D / 32) + db) * 2 * 64) * 8);
      base[r] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      base[32 + r] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      base[64 + r] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      base[96 + r] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

struct QArgs {
  const uint16_t *Q, *K, *V;
  const int32_t* perm;
  const float *rc, *rs;
  int N;
  uint32_t flags;
  float cL;
  uint8_t* Qq;
  float* sQ;
  uint8_t* Kq;
  float* sK;
  uint8_t* Vq;
  float* sV;
  uint16_t* mu;
  float* mu_scaled;
  uint16_t* mu_pack;
  dpair* ksum;
  float *vamax, *kbar, *vinv;
};

template <int D, bool ROPE, bool HAD, bool MX>
static void launch_quant(const QArgs& a, dim3 grid, int BH, hipStream_t st) {
  quant_stats<D, ROPE, HAD><<<grid, kQThreads, 0, st>>>(a.Q, a.K, a.V, a.perm, a.rc, a.rs, a.N, a.flags, a.cL, a.Qq,
                                                         a.sQ, a.mu, a.ksum, a.vamax);
  quant_reduce<D><<<dim3(BH, D / kRedCh), kQThreads, 0, st>>>(a.N, a.flags, a.ksum, a.vamax, a.kbar, a.sV, a.vinv);
  quant_apply<D, ROPE, HAD, MX><<<grid, kQThreads, 0, st>>>(a.K, a.V, a.perm, a.rc, a.rs, a.N, a.flags, a.kbar, a.sV,
                                                         a.vinv, a.mu, a.Kq, a.sK, a.Vq, a.mu_scaled, a.mu_pack);
}

}  // namespace vc

using namespace vc;

extern "C" int vc_launch_quantize(const void* Q, const void* K, const void* V, const int32_t* perm, const float* rc,
                                  const float* rs, int B, int H, int N, int d, uint32_t flags, float cL, uint8_t* Qq,
                                  float* sQ, uint8_t* Kq, float* sK, uint8_t* Vq, float* sV, void* mu, float* mu_scaled,
                                  void* mu_pack, void* ws, hipStream_t st) {
  const int nb = N / kBlock, BH = B * H;
  // workspace: ksum binary64 pairs [BH,nb,d] | vamax float [BH,nb,d] | kbar float [BH,d] | vinv float [BH,d] |
  // mu (if caller's NULL)
  char* w = (char*)ws;
  dpair* ksum = (dpair*)w; w += sizeof(dpair) * (size_t)BH * nb * d;
  float* vamax = (float*)w; w += sizeof(float) * (size_t)BH * nb * d;
  float* kbar = (float*)w; w += sizeof(float) * (size_t)BH * d;
  float* vinv = (float*)w; w += sizeof(float) * (size_t)BH * d;
  uint16_t* muw = (uint16_t*)w;
  uint16_t* mup = mu ? (uint16_t*)mu : muw;
  dim3 grid(nb, BH);
  const QArgs a{(const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, perm, rc, rs, N, flags, cL, Qq, sQ,
                Kq, sK, Vq, sV, mup, mu_scaled, (uint16_t*)mu_pack, ksum, vamax, kbar, vinv};
  const bool rope = rc != nullptr, had = (flags & kFlagHadamard) != 0, mx = (flags & kFlagMxfp4) != 0;
  const int sel = (rope ? 4 : 0) | (had ? 2 : 0) | (mx ? 1 : 0);
  if (d == 128) {
    switch (sel) {
      case 0: launch_quant<128, false, false, false>(a, grid, BH, st); break;
      case 1: launch_quant<128, false, false, true>(a, grid, BH, st); break;
      case 2: launch_quant<128, false, true, false>(a, grid, BH, st); break;
      case 3: launch_quant<128, false, true, true>(a, grid, BH, st); break;
      case 4: launch_quant<128, true, false, false>(a, grid, BH, st); break;
      case 5: launch_quant<128, true, false, true>(a, grid, BH, st); break;
      case 6: launch_quant<128, true, true, false>(a, grid, BH, st); break;
      default: launch_quant<128, true, true, true>(a, grid, BH, st); break;
    }
  } else {
    switch (sel) {
      case 0: launch_quant<64, false, false, false>(a, grid, BH, st); break;
      case 1: launch_quant<64, false, false, true>(a, grid, BH, st); break;
      case 2: launch_quant<64, false, true, false>(a, grid, BH, st); break;
      case 3: launch_quant<64, false, true, true>(a, grid, BH, st); break;
      case 4: launch_quant<64, true, false, false>(a, grid, BH, st); break;
      case 5: launch_quant<64, true, false, true>(a, grid, BH, st); break;
      case 6: launch_quant<64, true, true, false>(a, grid, BH, st); break;
      default: launch_quant<64, true, true, true>(a, grid, BH, st); break;
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" size_t vc_quantize_ws_bytes(int B, int H, int N, int d) {
  size_t BH = (size_t)B * H, nb = (size_t)N / kBlock;
  return sizeof(dpair) * BH * nb * d + sizeof(float) * BH * nb * d + 2 * sizeof(float) * BH * d +
         sizeof(uint16_t) * BH * nb * d + 256;
}
