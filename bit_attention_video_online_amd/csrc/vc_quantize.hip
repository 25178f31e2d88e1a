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
// All loads are 16-byte vectors of one token row; rows of V' and K' are gathered
// through pi. Exact sums use binary64, which is exact for these 128-term (or N-term)
// sums of bfloat16 values whenever their exponent span is moderate.
#include "vc_device.h"

namespace vc {

constexpr int kQThreads = 256;

// Block reduction of a float max over 256 threads (4 waves).
__device__ __forceinline__ float block_max_256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Quantise a [128 x D] tile held as rows of bf16 in `tile` (LDS, floats) with one
// scale; writes codes row-major to dst (global) and returns the scale.
template <int D>
__device__ __forceinline__ float quant_tile_rowmajor(const float* tile, uint8_t* dst, float* red) {
  constexpr int EL = kBlock * D;
  constexpr int STEPS = EL / (4 * kQThreads);  // float4 steps per thread: 16 (D=128) or 8 (D=64)
  const float4* t4 = reinterpret_cast<const float4*>(tile);
  float a = 0.0f;
  for (int i = 0; i < STEPS; i++) {
    float4 v = t4[i * kQThreads + threadIdx.x];
    a = fmaxf(fmaxf(fmaxf(a, fabsf(v.x)), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  }
  a = block_max_256(a, red);
  float s, inv;
  if (a > 0.0f) { s = a / 448.0f; inv = 448.0f / a; } else { s = 1.0f; inv = 0.0f; }
  uint32_t* o = reinterpret_cast<uint32_t*>(dst);
  for (int i = 0; i < STEPS; i++) {
    float4 v = t4[i * kQThreads + threadIdx.x];
    o[i * kQThreads + threadIdx.x] = e4m3x4_from_f32(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
  }
  return s;
}

// Load a 128-row tile of bf16 rows (rows gathered through `rows_of`, or contiguous)
// into LDS as floats. Thread layout: 16-byte vectors (8 bf16), D/8 vectors per row.
template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* base, const int32_t* perm_blk, float* tile, int nrows) {
  constexpr int VPR = D / 8;                 // vectors per row
  constexpr int NV = kBlock * VPR;           // vectors per tile
  for (int v = threadIdx.x; v < NV; v += kQThreads) {
    int r = v / VPR, c = (v % VPR) * 8;
    int src = perm_blk ? perm_blk[r] : r;
    src = ((unsigned)src < (unsigned)nrows) ? src : 0;  // a malformed permutation must not read out of bounds
    uint4 raw = *reinterpret_cast<const uint4*>(base + (size_t)src * D + c);
    float* t = tile + r * D + c;
    uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    for (int k = 0; k < 4; k++) {
      t[2 * k] = __uint_as_float(w[k] << 16);
      t[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kQThreads) void quant_stats(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                         int N, uint32_t flags, float cL,
                                                         uint8_t* __restrict__ Qq, float* __restrict__ sQ,
                                                         uint16_t* __restrict__ mu, double* __restrict__ ksum,
                                                         float* __restrict__ vamax) {
  __shared__ float tile[kBlock * D];
  __shared__ float red[4];
  __shared__ double part[kQThreads];
  const int nb = N / kBlock;
  const int j = blockIdx.x, bh = blockIdx.y;
  const size_t head = (size_t)bh * N * D;
  const int32_t* pblk = perm ? perm + (size_t)bh * N + (size_t)j * kBlock : nullptr;

  // ---- Q block (original order)
  load_rows<D>(Q + head + (size_t)j * kBlock * D, nullptr, tile, kBlock);
  __syncthreads();
  float s = quant_tile_rowmajor<D>(tile, Qq + head + (size_t)j * kBlock * D, red);
  if (threadIdx.x == 0) sQ[(size_t)bh * nb + j] = s * cL;
  __syncthreads();

  // ---- key channel partial sums (token order is irrelevant for a sum)
  constexpr int G = kQThreads / D;  // row groups: 2 (D=128) or 4 (D=64)
  const int c = threadIdx.x % D, g = threadIdx.x / D;
  if (flags & 1u) {
    load_rows<D>(K + head + (size_t)j * kBlock * D, nullptr, tile, kBlock);
    __syncthreads();
    double acc = 0.0;
    for (int r = g; r < kBlock; r += G) acc += (double)tile[r * D + c];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (g == 0) {
      double t = 0.0;
      for (int k = 0; k < G; k++) t += part[k * D + c];
      ksum[((size_t)bh * nb + j) * D + c] = t;
    }
    __syncthreads();
  }

  // ---- V' block: mean (bf16) and residual channel maximum
  if (pblk) load_rows<D>(V + head, pblk, tile, N);
  else load_rows<D>(V + head + (size_t)j * kBlock * D, nullptr, tile, kBlock);
  __syncthreads();
  float m = 0.0f;
  if (flags & 2u) {
    double acc = 0.0;
    for (int r = g; r < kBlock; r += G) acc += (double)tile[r * D + c];
    part[threadIdx.x] = acc;
    __syncthreads();
    double t = 0.0;
    for (int k = 0; k < G; k++) t += part[k * D + c];
    uint16_t h = f64_to_bf16(t * (1.0 / kBlock));
    m = bf16_to_f32(h);
    if (g == 0) mu[((size_t)bh * nb + j) * D + c] = h;
  } else if (mu != nullptr && g == 0) {
    mu[((size_t)bh * nb + j) * D + c] = 0;
  }
  float a = 0.0f;
  for (int r = g; r < kBlock; r += G) a = fmaxf(a, fabsf(tile[r * D + c] - m));
  __syncthreads();
  tile[threadIdx.x] = a;  // reuse: G partial maxima per channel
  __syncthreads();
  if (g == 0) {
    float t = 0.0f;
    for (int k = 0; k < G; k++) t = fmaxf(t, tile[k * D + c]);
    vamax[((size_t)bh * nb + j) * D + c] = t;
  }
}

template <int D>
__global__ __launch_bounds__(D) void quant_reduce(int N, uint32_t flags, const double* __restrict__ ksum,
                                                  const float* __restrict__ vamax, float* __restrict__ kbar,
                                                  float* __restrict__ sV, float* __restrict__ vinv) {
  const int nb = N / kBlock;
  const int bh = blockIdx.x, c = threadIdx.x;
  float kb = 0.0f;
  if (flags & 1u) {
    double t = 0.0;
    for (int j = 0; j < nb; j++) t += ksum[((size_t)bh * nb + j) * D + c];
    kb = div_to_f32(t, (double)N);
  }
  kbar[(size_t)bh * D + c] = kb;
  float a = 0.0f;
  for (int j = 0; j < nb; j++) a = fmaxf(a, vamax[((size_t)bh * nb + j) * D + c]);
  float s, inv;
  if (a > 0.0f) { s = a / 448.0f; inv = 448.0f / a; } else { s = 1.0f; inv = 0.0f; }
  sV[(size_t)bh * D + c] = s;
  vinv[(size_t)bh * D + c] = inv;
}

template <int D>
__global__ __launch_bounds__(kQThreads) void quant_apply(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                         const int32_t* __restrict__ perm, int N, uint32_t flags,
                                                         const float* __restrict__ kbar, const float* __restrict__ sV,
                                                         const float* __restrict__ vinv, const uint16_t* __restrict__ mu,
                                                         uint8_t* __restrict__ Kq, float* __restrict__ sK,
                                                         uint8_t* __restrict__ Vq, float* __restrict__ mu_scaled,
                                                         uint16_t* __restrict__ mu_pack) {
  __shared__ float tile[kBlock * D];
  __shared__ float red[4];
  __shared__ uint8_t codes[D * kBlock];
  const int nb = N / kBlock;
  const int j = blockIdx.x, bh = blockIdx.y;
  const size_t head = (size_t)bh * N * D;
  const int32_t* pblk = perm ? perm + (size_t)bh * N + (size_t)j * kBlock : nullptr;
  const size_t jrow = (size_t)j * kBlock * D;

  // ---- K~' = fl32(K[pi] - kbar), one scale per block, row-major codes
  if (pblk) load_rows<D>(K + head, pblk, tile, N);
  else load_rows<D>(K + head + jrow, nullptr, tile, kBlock);
  __syncthreads();
  {
    constexpr int EL = kBlock * D;
    for (int i = threadIdx.x; i < EL; i += kQThreads) tile[i] = tile[i] - kbar[(size_t)bh * D + (i % D)];
  }
  __syncthreads();
  float s = quant_tile_rowmajor<D>(tile, Kq + head + jrow, red);
  if (threadIdx.x == 0) sK[(size_t)bh * nb + j] = s;
  __syncthreads();

  // ---- residual codes of V'[block j], stored transposed: Vq[c][t]
  if (pblk) load_rows<D>(V + head, pblk, tile, N);
  else load_rows<D>(V + head + jrow, nullptr, tile, kBlock);
  __syncthreads();
  constexpr int G = kQThreads / D;
  const int c = threadIdx.x % D, g = threadIdx.x / D;
  const float m = (flags & 2u) ? bf16_to_f32(mu[((size_t)bh * nb + j) * D + c]) : 0.0f;
  const float inv = vinv[(size_t)bh * D + c];
  for (int r = g; r < kBlock; r += G) {
    float rr = tile[r * D + c] - m;
    codes[c * kBlock + r] = (uint8_t)e4m3_from_f32(rr * inv);
  }
  const float ms = (flags & 2u) ? m / sV[(size_t)bh * D + c] : 0.0f;
  if (g == 0 && mu_scaled) mu_scaled[((size_t)bh * nb + j) * D + c] = ms;
  if (g == 0 && mu_pack) {
    // mean-restoration operand, laid out as the A operands of two v_mfma_f32_32x32x16_bf16
    // per 32-channel block: [chunk of 8 key blocks][d-block][MFMA t][lane][8]. MFMA 0:
    // lanes 0-31 and 32-63 hold bf16(ms); MFMA 1: lanes 0-31 bf16(ms - bf16(ms)), lanes
    // 32-63 zero; lane l carries channel 32*d-block + l%32, element s key block 8*chunk + s.
    const int nc = (nb + 7) / 8, ch = j / 8, s8 = j % 8, db = c / 32, r = c % 32;
    const uint16_t hi = f32_to_bf16(ms);
    const uint16_t lo = f32_to_bf16(ms - bf16_to_f32(hi));
    uint16_t* base = mu_pack + ((((size_t)bh * nc + ch) * (D / 32) + db) * 2 * 64) * 8;
    base[(r) * 8 + s8] = hi;
    base[(32 + r) * 8 + s8] = hi;
    base[(64 + r) * 8 + s8] = lo;
    base[(96 + r) * 8 + s8] = 0;
    if (j == nb - 1) {  // key blocks past the end of the last chunk contribute nothing
      for (int t = s8 + 1; t < 8; t++) {
        base[(r) * 8 + t] = 0; base[(32 + r) * 8 + t] = 0; base[(64 + r) * 8 + t] = 0; base[(96 + r) * 8 + t] = 0;
      }
    }
  }
  __syncthreads();
  // contiguous copy-out of the D x 128 byte tile
  uint4* dst = reinterpret_cast<uint4*>(Vq + head + jrow);
  const uint4* srcv = reinterpret_cast<const uint4*>(codes);
  for (int i = threadIdx.x; i < D * kBlock / 16; i += kQThreads) dst[i] = srcv[i];
}

}  // namespace vc

using namespace vc;

extern "C" int vc_launch_quantize(const void* Q, const void* K, const void* V, const int32_t* perm, int B, int H, int N,
                                  int d, uint32_t flags, float cL, uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK,
                                  uint8_t* Vq, float* sV, void* mu, float* mu_scaled, void* mu_pack, void* ws,
                                  hipStream_t st) {
  const int nb = N / kBlock, BH = B * H;
  // workspace: ksum double [BH,nb,d] | vamax float [BH,nb,d] | kbar float [BH,d] | vinv float [BH,d] | mu (if caller's NULL)
  char* w = (char*)ws;
  double* ksum = (double*)w; w += sizeof(double) * (size_t)BH * nb * d;
  float* vamax = (float*)w; w += sizeof(float) * (size_t)BH * nb * d;
  float* kbar = (float*)w; w += sizeof(float) * (size_t)BH * d;
  float* vinv = (float*)w; w += sizeof(float) * (size_t)BH * d;
  uint16_t* muw = (uint16_t*)w;
  uint16_t* mup = mu ? (uint16_t*)mu : muw;
  dim3 grid(nb, BH);
  if (d == 128) {
    quant_stats<128><<<grid, kQThreads, 0, st>>>((const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, perm, N, flags, cL,
                                                Qq, sQ, mup, ksum, vamax);
    quant_reduce<128><<<BH, 128, 0, st>>>(N, flags, ksum, vamax, kbar, sV, vinv);
    quant_apply<128><<<grid, kQThreads, 0, st>>>((const uint16_t*)K, (const uint16_t*)V, perm, N, flags, kbar, sV, vinv, mup,
                                                Kq, sK, Vq, mu_scaled, (uint16_t*)mu_pack);
  } else {
    quant_stats<64><<<grid, kQThreads, 0, st>>>((const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, perm, N, flags, cL,
                                               Qq, sQ, mup, ksum, vamax);
    quant_reduce<64><<<BH, 64, 0, st>>>(N, flags, ksum, vamax, kbar, sV, vinv);
    quant_apply<64><<<grid, kQThreads, 0, st>>>((const uint16_t*)K, (const uint16_t*)V, perm, N, flags, kbar, sV, vinv, mup,
                                               Kq, sK, Vq, mu_scaled, (uint16_t*)mu_pack);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" size_t vc_quantize_ws_bytes(int B, int H, int N, int d) {
  size_t BH = (size_t)B * H, nb = (size_t)N / kBlock;
  return sizeof(double) * BH * nb * d + sizeof(float) * BH * nb * d + 2 * sizeof(float) * BH * d +
         sizeof(uint16_t) * BH * nb * d + 256;
}
