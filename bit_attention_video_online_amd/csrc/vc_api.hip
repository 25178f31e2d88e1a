// vc_api.hip -- the C ABI declared in include/vc.h: argument validation on the host, a check
// that the current device is a gfx950, then asynchronous launches on the caller's stream.
// Nothing here allocates or synchronises; the only state is a per-device record of the
// architecture check.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/vc.h"

extern "C" int vc_launch_quantize(const void* Q, const void* K, const void* V, const int32_t* perm, const float* rc,
                                  const float* rs, int B, int H, int N, int d, uint32_t flags, float cL, uint8_t* Qq,
                                  float* sQ, uint8_t* Kq, float* sK, uint8_t* Vq, float* sV, void* mu, float* mu_scaled,
                                  void* mu_pack, void* ws, hipStream_t st);
extern "C" size_t vc_quantize_ws_bytes(int B, int H, int N, int d);
extern "C" size_t vc_cluster_cost_ws_bytes(int B, int H, int N);
extern "C" int vc_launch_mfma_peak(int grid, int iters, int random_bits, float* out, hipStream_t st);
extern "C" int vc_launch_cluster_cost(const void* V, const float* C, const int32_t* labels, int B, int H, int N, int d,
                                      int K, double* cost, void* ws, hipStream_t st);
extern "C" int vc_launch_attention(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                                   const uint8_t* Vq, const float* sV, const void* mu_pack, int B, int H, int N, int d,
                                   float beta, int pmode, int mx, uint16_t* O, int dump_block, uint8_t* dump,
                                   hipStream_t st);
extern "C" int vc_launch_expcast(const float* acc, const float* s8, const float* bias, uint8_t* out, size_t n,
                                 int clamp, hipStream_t st);
extern "C" int vc_launch_mfma_f8_tiles(const uint8_t* A, const uint8_t* B, const float* C, float* D, int n,
                                       hipStream_t st);
extern "C" size_t vc_cluster_ws_bytes(int B, int H, int N, int d, int K);
extern "C" int vc_launch_cluster(const void* V, int B, int H, int N, int d, int K, int iters, int cold, float* C,
                                 int32_t* labels, int32_t* perm, void* ws, hipStream_t st, float lam, int32_t* nk_io);
extern "C" int vc_max_clusters(void);
extern "C" int vc_launch_exponent_span(const void* X, int kind, int BH, long long per_head, int32_t* out,
                                       hipStream_t st);
extern "C" int vc_launch_cluster_inc(const void* V, int B, int H, int N, int d, int K, float decay, int assign,
                                     float* C, float* M, int32_t* labels, int32_t* perm, void* ws, hipStream_t st);

namespace {

// fl32(log2(e) / sqrt(d)) for the supported head sizes, as exact binary32 bit patterns
// (log2(e)/8 and log2(e)/sqrt(128) rounded to nearest).
float log2e_over_sqrt_d(int d) {
  uint32_t bits = d == 64 ? 0x3e38aa3bu : 0x3e0293eeu;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

// B*H is a grid dimension of several kernels (at most 65535)
bool shape_ok(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (N % 128) != 0 || (d != 64 && d != 128)) return false;
  if ((long long)B * H > 65535) return false;
  const long long el = (long long)B * H * N * d;
  return el < (1LL << 31);
}
size_t vc_mu_pack_bytes(int B, int H, int N, int d) {
  const size_t nc = ((size_t)N / 128 + 7) / 8;
  return (size_t)B * H * nc * (d / 16) * 64 * 8 * 2;
}
bool aligned16(const void* p) { return p == nullptr || (((uintptr_t)p) & 15u) == 0; }

struct Range {
  const char* a;
  size_t n;
};
bool overlaps(Range x, Range y) {
  if (!x.a || !y.a || x.n == 0 || y.n == 0) return false;
  return x.a < y.a + y.n && y.a < x.a + x.n;
}

// The current device must be a gfx950 (the kernels are built for it alone). The answer is
// kept per device ordinal; concurrent first calls may both query, and write the same value.
vc_status device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();  // leave no sticky error behind for the caller
    return VC_E_UNSUPPORTED;
  }
  static int known[64];  // 0 unknown, 1 gfx950, 2 other
  if (dev < 64 && known[dev]) return known[dev] == 1 ? VC_OK : VC_E_UNSUPPORTED;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return VC_E_UNSUPPORTED;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) known[dev] = ok ? 1 : 2;
  return ok ? VC_OK : VC_E_UNSUPPORTED;
}

}  // namespace

extern "C" const char* vc_status_string(vc_status s) {
  switch (s) {
    case VC_OK: return "VC_OK";
    case VC_E_NULLPTR: return "VC_E_NULLPTR: a required pointer is NULL";
    case VC_E_SHAPE: return "VC_E_SHAPE: need B,H >= 1, N a positive multiple of 128, d in {64,128}, block 128";
    case VC_E_PARAM: return "VC_E_PARAM: cluster count, iterations, beta or flags out of range";
    case VC_E_WORKSPACE: return "VC_E_WORKSPACE: workspace smaller than required";
    case VC_E_UNSUPPORTED: return "VC_E_UNSUPPORTED: misaligned buffer or unsupported device";
    case VC_E_HIP: return "VC_E_HIP: a HIP launch failed";
    case VC_E_ALIAS: return "VC_E_ALIAS: an output overlaps an input";
    default: return "unknown vc_status";
  }
}

extern "C" int vc_abi_version(void) { return VC_ABI_VERSION; }

extern "C" size_t vc_cluster_workspace_bytes(int B, int H, int N, int d, int K) {
  if (!shape_ok(B, H, N, d) || K < 1 || K > N) return 0;
  return vc_cluster_ws_bytes(B, H, N, d, K);
}

extern "C" vc_status vc_cluster(const void* V, int B, int H, int N, int d, int K, int iters, int cold_start,
                                float* centroids, int32_t* labels, int32_t* perm, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!V || !centroids || !labels || !perm || !workspace) return VC_E_NULLPTR;
  if (!shape_ok(B, H, N, d)) return VC_E_SHAPE;
  if (K < 1 || K > N || K > vc_max_clusters() || iters < 1 || iters > 1000) return VC_E_PARAM;
  if (workspace_bytes < vc_cluster_ws_bytes(B, H, N, d, K)) return VC_E_WORKSPACE;
  if (!aligned16(V) || !aligned16(centroids) || !aligned16(labels) || !aligned16(perm) || !aligned16(workspace))
    return VC_E_UNSUPPORTED;
  const size_t el = (size_t)B * H * N;
  Range in{(const char*)V, el * d * 2};
  if (overlaps(in, {(const char*)centroids, (size_t)B * H * K * d * 4}) || overlaps(in, {(const char*)labels, el * 4}) ||
      overlaps(in, {(const char*)perm, el * 4}) || overlaps({(const char*)labels, el * 4}, {(const char*)perm, el * 4}))
    return VC_E_ALIAS;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_cluster(V, B, H, N, d, K, iters, cold_start ? 1 : 0, centroids, labels, perm, workspace,
                        (hipStream_t)stream, 0.0f, nullptr) != 0)
    return VC_E_HIP;
  return VC_OK;
}

extern "C" vc_status vc_cluster_balanced(const void* V, int B, int H, int N, int d, int K, int iters, int cold_start,
                                         float lambda, int32_t* counts, float* centroids, int32_t* labels,
                                         int32_t* perm, void* workspace, size_t workspace_bytes, void* stream) {
  if (!V || !counts || !centroids || !labels || !perm || !workspace) return VC_E_NULLPTR;
  if (!shape_ok(B, H, N, d)) return VC_E_SHAPE;
  if (K < 1 || K > N || K > vc_max_clusters() || iters < 1 || iters > 1000) return VC_E_PARAM;
  if (!(lambda >= 0.0f) || !(lambda < __builtin_inff())) return VC_E_PARAM;
  if (workspace_bytes < vc_cluster_ws_bytes(B, H, N, d, K)) return VC_E_WORKSPACE;
  if (!aligned16(V) || !aligned16(centroids) || !aligned16(labels) || !aligned16(perm) || !aligned16(workspace) ||
      !aligned16(counts))
    return VC_E_UNSUPPORTED;
  const size_t el = (size_t)B * H * N;
  const Range outs[] = {{(const char*)centroids, (size_t)B * H * K * d * 4}, {(const char*)labels, el * 4},
                        {(const char*)perm, el * 4}, {(const char*)counts, (size_t)B * H * K * 4},
                        {(const char*)workspace, workspace_bytes}};
  const Range in{(const char*)V, el * d * 2};
  for (int i = 0; i < 5; i++) {
    if (overlaps(in, outs[i])) return VC_E_ALIAS;
    for (int j = i + 1; j < 5; j++)
      if (overlaps(outs[i], outs[j])) return VC_E_ALIAS;
  }
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_cluster(V, B, H, N, d, K, iters, cold_start ? 1 : 0, centroids, labels, perm, workspace,
                        (hipStream_t)stream, lambda, counts) != 0)
    return VC_E_HIP;
  return VC_OK;
}

extern "C" vc_status vc_cluster_incremental(const void* V, int B, int H, int N, int d, int K, float decay, int assign,
                                            float* centroids, float* mass, int32_t* labels, int32_t* perm,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!V || !centroids || !mass || !labels || !perm || !workspace) return VC_E_NULLPTR;
  if (!shape_ok(B, H, N, d)) return VC_E_SHAPE;
  if (K < 1 || K > N || K > vc_max_clusters()) return VC_E_PARAM;
  if (!(decay >= 0.0f && decay <= 1.0f)) return VC_E_PARAM;  // also rejects NaN
  if (workspace_bytes < vc_cluster_ws_bytes(B, H, N, d, K)) return VC_E_WORKSPACE;
  const void* ptrs[] = {V, centroids, mass, labels, perm, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return VC_E_UNSUPPORTED;
  const size_t el = (size_t)B * H * N;
  const Range in{(const char*)V, el * d * 2};
  const Range bufs[] = {{(const char*)centroids, (size_t)B * H * K * d * 4}, {(const char*)mass, (size_t)B * H * K * 4},
                        {(const char*)labels, el * 4}, {(const char*)perm, el * 4},
                        {(const char*)workspace, workspace_bytes}};
  for (int i = 0; i < 5; i++) {
    if (overlaps(in, bufs[i])) return VC_E_ALIAS;
    for (int j = i + 1; j < 5; j++)
      if (overlaps(bufs[i], bufs[j])) return VC_E_ALIAS;
  }
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_cluster_inc(V, B, H, N, d, K, decay, assign ? 1 : 0, centroids, mass, labels, perm, workspace,
                            (hipStream_t)stream) != 0)
    return VC_E_HIP;
  return VC_OK;
}

extern "C" size_t vc_cluster_cost_workspace_bytes(int B, int H, int N, int d) {
  if (!shape_ok(B, H, N, d)) return 0;
  return vc_cluster_cost_ws_bytes(B, H, N);
}

extern "C" vc_status vc_cluster_cost(const void* V, const float* centroids, const int32_t* labels, int B, int H, int N,
                                     int d, int K, double* cost, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!V || !centroids || !labels || !cost || !workspace) return VC_E_NULLPTR;
  if (!shape_ok(B, H, N, d)) return VC_E_SHAPE;
  if (K < 1 || K > N) return VC_E_PARAM;
  if (workspace_bytes < vc_cluster_cost_ws_bytes(B, H, N)) return VC_E_WORKSPACE;
  if (!aligned16(V) || !aligned16(centroids) || !aligned16(labels) || !aligned16(workspace)) return VC_E_UNSUPPORTED;
  if (((uintptr_t)cost) & 7u) return VC_E_UNSUPPORTED;
  const size_t el = (size_t)B * H * N;
  const Range outs[] = {{(const char*)cost, (size_t)B * H * 8}, {(const char*)workspace, workspace_bytes}};
  const Range ins[] = {{(const char*)V, el * d * 2}, {(const char*)centroids, (size_t)B * H * K * d * 4},
                       {(const char*)labels, el * 4}};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o, i)) return VC_E_ALIAS;
  if (overlaps(outs[0], outs[1])) return VC_E_ALIAS;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_cluster_cost(V, centroids, labels, B, H, N, d, K, cost, workspace, (hipStream_t)stream) != 0)
    return VC_E_HIP;
  return VC_OK;
}

extern "C" vc_status vc_exponent_span(const void* X, int kind, int B, int H, int rows, int d, int32_t* out,
                                      void* stream) {
  if (!X || !out) return VC_E_NULLPTR;
  if (kind < 0 || kind > 2) return VC_E_PARAM;
  if (B < 1 || H < 1 || rows < 1 || d < 1 || (long long)B * H > 65535) return VC_E_SHAPE;
  const long long per_head = (long long)rows * d;
  if ((long long)B * H * per_head >= (1LL << 31)) return VC_E_SHAPE;
  const size_t esz = kind == 0 ? 2 : 4;
  if ((((uintptr_t)X) & (esz - 1)) || (((uintptr_t)out) & 3u)) return VC_E_UNSUPPORTED;
  const Range o{(const char*)out, (size_t)B * H * 2 * sizeof(int32_t)};
  const Range i{(const char*)X, (size_t)(B * (long long)H * per_head) * esz};
  if (overlaps(o, i)) return VC_E_ALIAS;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_exponent_span(X, kind, B * H, per_head, out, (hipStream_t)stream) != 0) return VC_E_HIP;
  return VC_OK;
}

extern "C" size_t vc_mu_pack_size(int B, int H, int N, int d) {
  if (!shape_ok(B, H, N, d)) return 0;
  return vc_mu_pack_bytes(B, H, N, d);
}

extern "C" size_t vc_quantize_workspace_bytes(int B, int H, int N, int d, int block) {
  if (!shape_ok(B, H, N, d) || block != 128) return 0;
  return vc_quantize_ws_bytes(B, H, N, d);
}

// ---- the allocation-free quantiser: the workspace that vc_quantize takes from its caller lives
// in a file-scope device array instead. Every device that runs it holds its own copy until the
// process ends; the host-side name is only a stand-in, so the array is always addressed through
// the device address hipGetSymbolAddress returns for the current device (kept per ordinal).
static __device__ __align__(256) unsigned char scratch[VC_QUANTIZE_NOALLOC_SCRATCH_BYTES];
static void* scratch_dev[64];

static vc_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return VC_E_UNSUPPORTED;
  }
  if (!scratch_dev[dev]) {  // first call on this device (concurrent first calls store the same value)
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return VC_E_HIP;
    }
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return VC_OK;
}

static vc_status quantize_common(const void* Q, const void* K, const void* V, const int32_t* perm,
                                 const float* rope_cos, const float* rope_sin, int B, int H, int N, int d, int block,
                                 uint32_t flags, uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK, uint8_t* Vq,
                                 float* sV, void* mu, float* mu_scaled, void* mu_pack, void* workspace,
                                 size_t workspace_bytes, void* stream, bool noalloc = false) {
  if (!Q || !K || !V || !Qq || !sQ || !Kq || !sK || !Vq || !sV || (!workspace && !noalloc)) return VC_E_NULLPTR;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return VC_E_NULLPTR;
  if (!shape_ok(B, H, N, d) || block != 128) return VC_E_SHAPE;
  if (flags & ~(uint32_t)(VC_F_KSMOOTH | VC_F_VSMOOTH | VC_F_EXPCAST | VC_F_HADAMARD | VC_F_MXFP4)) return VC_E_PARAM;
  const size_t need = vc_quantize_ws_bytes(B, H, N, d);
  if (noalloc ? need > (size_t)VC_QUANTIZE_NOALLOC_SCRATCH_BYTES : workspace_bytes < need) return VC_E_WORKSPACE;
  const void* ptrs[] = {Q, K, V, perm, rope_cos, rope_sin, Qq, sQ, Kq, sK, Vq, sV, mu, mu_scaled, mu_pack, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return VC_E_UNSUPPORTED;
  const size_t el = (size_t)B * H * N * d, nbk = (size_t)B * H * (N / 128);
  const size_t tab = (size_t)N * (d / 2) * 4;
  const Range ins[] = {{(const char*)Q, el * 2}, {(const char*)K, el * 2}, {(const char*)V, el * 2},
                       {(const char*)perm, (size_t)B * H * N * 4}, {(const char*)rope_cos, tab},
                       {(const char*)rope_sin, tab}};
  const Range outs[] = {{(const char*)Qq, el}, {(const char*)sQ, nbk * 4}, {(const char*)Kq, el},
                        {(const char*)sK, nbk * 4}, {(const char*)Vq, el}, {(const char*)sV, (size_t)B * H * d * 4},
                        {(const char*)mu, nbk * d * 2}, {(const char*)mu_scaled, nbk * d * 4},
                        {(const char*)mu_pack, vc_mu_pack_bytes(B, H, N, d)}};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o, i)) return VC_E_ALIAS;
  if (const vc_status dc = device_check()) return dc;
  void* ws = workspace;
  if (noalloc)
    if (const vc_status sp = scratch_ptr(&ws)) return sp;
  if (vc_launch_quantize(Q, K, V, perm, rope_cos, rope_sin, B, H, N, d, flags, log2e_over_sqrt_d(d), Qq, sQ, Kq, sK,
                         Vq, sV, mu, mu_scaled, mu_pack, ws, (hipStream_t)stream) != 0)
    return VC_E_HIP;
  return VC_OK;
}

extern "C" vc_status vc_quantize(const void* Q, const void* K, const void* V, const int32_t* perm, int B, int H, int N,
                                 int d, int block, uint32_t flags, uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK,
                                 uint8_t* Vq, float* sV, void* mu, float* mu_scaled, void* mu_pack, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return quantize_common(Q, K, V, perm, nullptr, nullptr, B, H, N, d, block, flags, Qq, sQ, Kq, sK, Vq, sV, mu,
                         mu_scaled, mu_pack, workspace, workspace_bytes, stream);
}

extern "C" vc_status vc_quantize_noalloc(const void* Q, const void* K, const void* V, const int32_t* perm, int B,
                                         int H, int N, int d, int block, uint32_t flags, uint8_t* Qq, float* sQ,
                                         uint8_t* Kq, float* sK, uint8_t* Vq, float* sV, void* mu, float* mu_scaled,
                                         void* mu_pack, void* stream) {
  return quantize_common(Q, K, V, perm, nullptr, nullptr, B, H, N, d, block, flags, Qq, sQ, Kq, sK, Vq, sV, mu,
                         mu_scaled, mu_pack, nullptr, 0, stream, true);
}

extern "C" vc_status vc_quantize_rope(const void* Q, const void* K, const void* V, const int32_t* perm,
                                      const float* rope_cos, const float* rope_sin, int B, int H, int N, int d,
                                      int block, uint32_t flags, uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK,
                                      uint8_t* Vq, float* sV, void* mu, float* mu_scaled, void* mu_pack,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!rope_cos || !rope_sin) return VC_E_NULLPTR;
  return quantize_common(Q, K, V, perm, rope_cos, rope_sin, B, H, N, d, block, flags, Qq, sQ, Kq, sK, Vq, sV, mu,
                         mu_scaled, mu_pack, workspace, workspace_bytes, stream);
}

static vc_status attention_common(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                                  const uint8_t* Vq, const float* sV, const void* mu_pack, int B, int H, int N, int d,
                                  int block, float beta, uint32_t flags, void* O, int dump_block, uint8_t* codes,
                                  void* stream) {
  if (!Qq || !sQ || !Kq || !sK || !Vq || !sV || !O) return VC_E_NULLPTR;
  if (!shape_ok(B, H, N, d) || block != 128) return VC_E_SHAPE;
  if (!isfinite(beta) ||
      (flags & ~(uint32_t)(VC_F_KSMOOTH | VC_F_VSMOOTH | VC_F_EXPCAST | VC_F_E5M2 | VC_F_MXFP4)))
    return VC_E_PARAM;
  if ((flags & VC_F_E5M2) && !(flags & VC_F_EXPCAST)) return VC_E_PARAM;  // E5M2 bytes exist only as ExpCast
  const void* ptrs[] = {Qq, sQ, Kq, sK, Vq, sV, mu_pack, O, codes};
  for (const void* p : ptrs)
    if (!aligned16(p)) return VC_E_UNSUPPORTED;
  const size_t el = (size_t)B * H * N * d, nbk = (size_t)B * H * (N / 128);
  const Range ins[] = {{(const char*)Qq, el}, {(const char*)sQ, nbk * 4}, {(const char*)Kq, el},
                       {(const char*)sK, nbk * 4}, {(const char*)Vq, el}, {(const char*)sV, (size_t)B * H * d * 4},
                       {(const char*)mu_pack, vc_mu_pack_bytes(B, H, N, d)}};
  const Range outs[] = {{(const char*)O, el * 2}, {(const char*)codes, (size_t)B * H * N * 128}};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlaps(o, i)) return VC_E_ALIAS;
  if (overlaps(outs[0], outs[1])) return VC_E_ALIAS;
  const int pmode = (flags & VC_F_EXPCAST) ? ((flags & VC_F_E5M2) ? 2 : 1) : 0;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_attention(Qq, sQ, Kq, sK, Vq, sV, mu_pack, B, H, N, d, beta, pmode, (flags & VC_F_MXFP4) ? 1 : 0,
                          (uint16_t*)O, dump_block, codes, (hipStream_t)stream) != 0)
    return VC_E_HIP;
  return VC_OK;
}

extern "C" vc_status vc_attention(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                                  const uint8_t* Vq, const float* sV, const void* mu_pack, int B, int H, int N, int d,
                                  int block, float beta, uint32_t flags, void* O, void* stream) {
  return attention_common(Qq, sQ, Kq, sK, Vq, sV, mu_pack, B, H, N, d, block, beta, flags, O, -1, nullptr, stream);
}

extern "C" vc_status vc_attention_dump(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                                       const uint8_t* Vq, const float* sV, const void* mu_pack, int B, int H, int N,
                                       int d, int block, float beta, uint32_t flags, void* O, int dump_block,
                                       uint8_t* codes, void* stream) {
  if (!codes) return VC_E_NULLPTR;
  if (N >= 128 && (dump_block < 0 || dump_block >= N / 128)) return VC_E_PARAM;
  return attention_common(Qq, sQ, Kq, sK, Vq, sV, mu_pack, B, H, N, d, block, beta, flags, O, dump_block, codes,
                          stream);
}

extern "C" vc_status vc_debug_mfma_peak(int grid, int iters, int random_bits, float* out, void* stream) {
  if (!out) return VC_E_NULLPTR;
  if (grid < 1 || iters < 1) return VC_E_PARAM;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_mfma_peak(grid, iters, random_bits ? 1 : 0, out, (hipStream_t)stream) != 0) return VC_E_HIP;
  return VC_OK;
}

static vc_status debug_expcast(const float* acc, const float* scale8, const float* bias, uint8_t* codes, size_t n,
                               int clamp, void* stream) {
  if (n == 0) return VC_OK;
  if (!acc || !scale8 || !bias || !codes) return VC_E_NULLPTR;
  if (n > ((size_t)1 << 34)) return VC_E_PARAM;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_expcast(acc, scale8, bias, codes, n, clamp, (hipStream_t)stream) != 0) return VC_E_HIP;
  return VC_OK;
}

extern "C" vc_status vc_debug_expcast(const float* acc, const float* scale8, const float* bias, uint8_t* codes, size_t n,
                                      void* stream) {
  return debug_expcast(acc, scale8, bias, codes, n, 1, stream);
}

extern "C" vc_status vc_debug_expcast_unclamped(const float* acc, const float* scale8, const float* bias,
                                                uint8_t* codes, size_t n, void* stream) {
  return debug_expcast(acc, scale8, bias, codes, n, 0, stream);
}

extern "C" vc_status vc_debug_mfma_f8(const uint8_t* A, const uint8_t* B, const float* C, float* D, int ntiles,
                                      void* stream) {
  if (ntiles == 0) return VC_OK;
  if (!A || !B || !C || !D) return VC_E_NULLPTR;
  if (ntiles < 0 || ntiles > (1 << 20)) return VC_E_PARAM;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(D)) return VC_E_UNSUPPORTED;
  const size_t n = (size_t)ntiles;
  const Range outs{(const char*)D, n * 4096};
  if (overlaps(outs, {(const char*)A, n * 2048}) || overlaps(outs, {(const char*)B, n * 2048}) ||
      overlaps(outs, {(const char*)C, n * 4096}))
    return VC_E_ALIAS;
  if (const vc_status dc = device_check()) return dc;
  if (vc_launch_mfma_f8_tiles(A, B, C, D, ntiles, (hipStream_t)stream) != 0) return VC_E_HIP;
  return VC_OK;
}
