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
//   cl_prep    chat = bf16(C) (as binary32), |chat|^2
//   cl_assign  distances |c|^2 - 2 v.c in binary32 over a 64-token x 64-centroid LDS
//              tile, with a rigorous per-distance error bound; a token whose best
//              candidate is not separated from the rest by the bounds is re-ranked
//              in binary64 (exact for bf16 data of moderate dynamic range).
//   cl_hist / cl_scan / cl_scatter   stable counting sort of the labels (pi)
//   cl_update  C_k = fl32(sum of members / count), binary64 sums in pi order
// No atomics on floating-point data: every result is run-to-run deterministic.
#include "vc_device.h"

namespace vc {

constexpr int kTok = 64;      // tokens per assign tile
constexpr int kCen = 64;      // centroids per assign chunk
constexpr int kChunk = 256;   // tokens per sort chunk
constexpr int kMaxClusters = 8192;

__global__ void cl_cold(const uint16_t* __restrict__ V, float* __restrict__ C, int N, int K, int D) {
  const int k = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const long long t = ((long long)(2 * k + 1) * N) / (2LL * K);
  C[((size_t)bh * K + k) * D + c] = bf16_to_f32(V[((size_t)bh * N + t) * D + c]);
}

__global__ void cl_prep(const float* __restrict__ C, float* __restrict__ chat, float* __restrict__ cnorm, int K, int D) {
  __shared__ double part[128];
  const int k = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const size_t o = ((size_t)bh * K + k) * D + c;
  const float h = bf16_to_f32(f32_to_bf16(C[o]));
  chat[o] = h;
  part[c] = (double)h * (double)h;  // exact square of a bf16 value
  __syncthreads();
  if (c == 0) {
    double s = 0.0;
    for (int i = 0; i < D; i++) s += part[i];
    cnorm[(size_t)bh * K + k] = (float)s;
  }
}

// record for the per-token best / bound tracking
struct Cand {
  float d;   // best distance' (|c|^2 - 2 v.c)
  float e;   // its error bound
  float lb;  // min over the other clusters of (distance' - bound)
  int k;
};

__device__ __forceinline__ void cand_push(Cand& c, float d, float e, int k) {
  if (d < c.d || (d == c.d && k < c.k)) {
    c.lb = fminf(c.lb, c.d - c.e);
    c.d = d; c.e = e; c.k = k;
  } else {
    c.lb = fminf(c.lb, d - e);
  }
}
__device__ __forceinline__ void cand_merge(Cand& a, const Cand& b) {
  if (b.d < a.d || (b.d == a.d && b.k < a.k)) {
    float lb = fminf(fminf(a.lb, b.lb), a.d - a.e);
    a.d = b.d; a.e = b.e; a.k = b.k; a.lb = lb;
  } else {
    a.lb = fminf(fminf(a.lb, b.lb), b.d - b.e);
  }
}

template <int D>
__global__ __launch_bounds__(256) void cl_assign(const uint16_t* __restrict__ V, const float* __restrict__ chat,
                                                 const float* __restrict__ cnorm, int N, int K,
                                                 int32_t* __restrict__ labels) {
  __shared__ __attribute__((aligned(16))) float Vt[D][kTok];   // transposed token tile
  __shared__ __attribute__((aligned(16))) float Ct[D][kCen];   // transposed centroid chunk
  __shared__ float vnorm[kTok];
  __shared__ float cn[kCen];
  __shared__ Cand rec[kTok][16];
  __shared__ int unsure[kTok];
  __shared__ int n_unsure;
  __shared__ double red_d[256];
  __shared__ int red_k[256];

  const int bh = blockIdx.y, t0 = blockIdx.x * kTok;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const uint16_t* Vh = V + (size_t)bh * N * D;
  const float* Ch = chat + (size_t)bh * K * D;
  const float* Nh = cnorm + (size_t)bh * K;
  const int ntok = min(kTok, N - t0);

  // token tile (transposed) and token norms
  for (int i = tid; i < kTok * D; i += 256) {
    int t = i / D, c = i % D;
    Vt[c][t] = (t < ntok) ? bf16_to_f32(Vh[(size_t)(t0 + t) * D + c]) : 0.0f;
  }
  __syncthreads();
  if (tid < kTok) {
    float s = 0.0f;
    for (int c = 0; c < D; c++) s = __builtin_fmaf(Vt[c][tid], Vt[c][tid], s);
    vnorm[tid] = sqrtf(s) * 1.0001f;  // upper bound of |v|
  }
  const float u = 5.9604645e-8f;                    // 2^-24
  const float gam = (float)D * u / (1.0f - (float)D * u);

  Cand cand[4];
  for (int i = 0; i < 4; i++) cand[i] = Cand{__builtin_inff(), 0.0f, __builtin_inff(), 0x7fffffff};

  for (int k0 = 0; k0 < K; k0 += kCen) {
    __syncthreads();
    for (int i = tid; i < kCen * D; i += 256) {
      int k = i / D, c = i % D;
      Ct[c][k] = (k0 + k < K) ? Ch[(size_t)(k0 + k) * D + c] : 0.0f;
    }
    if (tid < kCen) cn[tid] = (k0 + tid < K) ? Nh[k0 + tid] : 0.0f;
    __syncthreads();
    float dot[4][4];
    for (int i = 0; i < 4; i++)
      for (int k = 0; k < 4; k++) dot[i][k] = 0.0f;
    for (int c = 0; c < D; c++) {
      const float4 v4 = *reinterpret_cast<const float4*>(&Vt[c][ty * 4]);
      const float4 c4 = *reinterpret_cast<const float4*>(&Ct[c][tx * 4]);
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
      const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
      for (int i = 0; i < 4; i++)
        for (int k = 0; k < 4; k++) dot[i][k] = __builtin_fmaf(vv[i], cc[k], dot[i][k]);
    }
    for (int k = 0; k < 4; k++) {
      const int kk = k0 + tx * 4 + k;
      if (kk >= K) continue;
      const float cnk = cn[tx * 4 + k];
      const float cabs = sqrtf(cnk) * 1.0001f;
      for (int i = 0; i < 4; i++) {
        const float dd = cnk - 2.0f * dot[i][k];
        const float e = 2.0f * (2.0f * gam * vnorm[ty * 4 + i] * cabs + u * (cnk + fabsf(dd))) + 1e-30f;
        cand_push(cand[i], dd, e, kk);
      }
    }
  }
  // merge the 16 partial records of each token
  for (int i = 0; i < 4; i++) rec[ty * 4 + i][tx] = cand[i];
  if (tid == 0) n_unsure = 0;
  __syncthreads();
  if (tid < kTok && tid < ntok) {
    Cand a = rec[tid][0];
    for (int x = 1; x < 16; x++) cand_merge(a, rec[tid][x]);
    if (a.lb > a.d + a.e) {
      labels[(size_t)bh * N + t0 + tid] = ((unsigned)a.k < (unsigned)K) ? a.k : 0;
    } else {
      int slot = atomicAdd(&n_unsure, 1);
      unsure[slot] = tid;
    }
  }
  __syncthreads();
  // exact re-rank (binary64) of the uncertain tokens, the whole group per token
  const int nu = n_unsure;
  for (int ui = 0; ui < nu; ui++) {
    const int t = unsure[ui];
    double best = __builtin_inf();
    int bk = 0x7fffffff;
    for (int k = tid; k < K; k += 256) {
      const float* ck = Ch + (size_t)k * D;
      double s = 0.0;
      for (int c = 0; c < D; c++) {
        double df = (double)Vt[c][t] - (double)ck[c];
        s = fma(df, df, s);
      }
      if (s < best) { best = s; bk = k; }  // k ascending per thread: ties keep the lower
    }
    red_d[tid] = best;
    red_k[tid] = bk;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        double d2 = red_d[tid + o];
        int k2 = red_k[tid + o];
        if (d2 < red_d[tid] || (d2 == red_d[tid] && k2 < red_k[tid])) { red_d[tid] = d2; red_k[tid] = k2; }
      }
      __syncthreads();
    }
    if (tid == 0) labels[(size_t)bh * N + t0 + t] = ((unsigned)red_k[0] < (unsigned)K) ? red_k[0] : 0;
    __syncthreads();
  }
}

// counts[bh][k][chunk]
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
  for (int k = threadIdx.x; k < K; k += 256) counts[((size_t)bh * K + k) * nch + ch] = hist[k];
}

// exclusive scan of counts in (k, chunk) order per head; cluster starts and sizes
__global__ __launch_bounds__(1024) void cl_scan(const int32_t* __restrict__ counts, int K, int nch,
                                                int32_t* __restrict__ offsets, int32_t* __restrict__ cstart,
                                                int32_t* __restrict__ csize) {
  __shared__ int part[1024];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const size_t total = (size_t)K * nch;
  const size_t per = (total + 1023) / 1024;
  const size_t a = tid * per, b = min(total, a + per);
  const int32_t* cnt = counts + (size_t)bh * total;
  int32_t* off = offsets + (size_t)bh * total;
  int s = 0;
  for (size_t i = a; i < b; i++) s += cnt[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    int v = (tid >= o) ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;  // exclusive prefix of this thread's range
  for (size_t i = a; i < b; i++) {
    off[i] = run;
    run += cnt[i];
  }
  __syncthreads();
  for (int k = tid; k < K; k += 1024) {
    cstart[(size_t)bh * K + k] = off[(size_t)k * nch];
    int z = 0;
    for (int c = 0; c < nch; c++) z += cnt[(size_t)k * nch + c];
    csize[(size_t)bh * K + k] = z;
  }
}

__global__ __launch_bounds__(256) void cl_scatter(const int32_t* __restrict__ labels, int N, int K, int nch,
                                                  const int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
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
    perm[(size_t)bh * N + offsets[((size_t)bh * K + z) * nch + ch] + rank] = t;
  }
}

__global__ void cl_update(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                          const int32_t* __restrict__ cstart, const int32_t* __restrict__ csize, int N, int K, int D,
                          float* __restrict__ C) {
  const int k = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const int n = csize[(size_t)bh * K + k];
  if (n == 0) return;  // empty cluster keeps its centroid
  const int s0 = cstart[(size_t)bh * K + k];
  const uint16_t* Vh = V + (size_t)bh * N * D;
  const int32_t* ph = perm + (size_t)bh * N;
  double s = 0.0;
  for (int i = 0; i < n; i++) s += (double)bf16_to_f32(Vh[(size_t)ph[s0 + i] * D + c]);
  C[((size_t)bh * K + k) * D + c] = div_to_f32(s, (double)n);
}

}  // namespace vc

using namespace vc;

extern "C" size_t vc_cluster_ws_bytes(int B, int H, int N, int d, int K) {
  const size_t BH = (size_t)B * H, nch = ((size_t)N + kChunk - 1) / kChunk;
  return BH * K * d * sizeof(float) + BH * K * sizeof(float) + 2 * BH * K * nch * sizeof(int32_t) +
         2 * BH * K * sizeof(int32_t) + 1024;
}

extern "C" int vc_launch_cluster(const void* Vv, int B, int H, int N, int d, int K, int iters, int cold, float* C,
                                 int32_t* labels, int32_t* perm, void* ws, hipStream_t st) {
  const uint16_t* V = (const uint16_t*)Vv;
  const int BH = B * H, nch = (N + kChunk - 1) / kChunk;
  char* w = (char*)ws;
  float* chat = (float*)w; w += (size_t)BH * K * d * sizeof(float);
  float* cnorm = (float*)w; w += (size_t)BH * K * sizeof(float);
  int32_t* counts = (int32_t*)w; w += (size_t)BH * K * nch * sizeof(int32_t);
  int32_t* offs = (int32_t*)w; w += (size_t)BH * K * nch * sizeof(int32_t);
  int32_t* cstart = (int32_t*)w; w += (size_t)BH * K * sizeof(int32_t);
  int32_t* csize = (int32_t*)w;
  if (cold) cl_cold<<<dim3(K, BH), d, 0, st>>>(V, C, N, K, d);
  const dim3 gtok((N + kTok - 1) / kTok, BH), gch(nch, BH), gk(K, BH);
  for (int it = 0; it < iters; it++) {
    cl_prep<<<gk, d, 0, st>>>(C, chat, cnorm, K, d);
    if (d == 128) cl_assign<128><<<gtok, 256, 0, st>>>(V, chat, cnorm, N, K, labels);
    else cl_assign<64><<<gtok, 256, 0, st>>>(V, chat, cnorm, N, K, labels);
    cl_hist<<<gch, 256, K * sizeof(int), st>>>(labels, N, K, nch, counts);
    cl_scan<<<BH, 1024, 0, st>>>(counts, K, nch, offs, cstart, csize);
    cl_scatter<<<gch, 256, 0, st>>>(labels, N, K, nch, offs, perm);
    cl_update<<<gk, d, 0, st>>>(V, perm, cstart, csize, N, K, d, C);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int vc_max_clusters(void) { return kMaxClusters; }
