/*
 * vc.h -- C ABI of the VC-Attention hot path for AMD Instinct MI355X (gfx950).
 *
 * Method: "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
 * Attention" (arXiv 2609.15810). Non-causal FP8 flash attention with
 *   - V-Smooth: online k-means on value tokens per (batch, head), one joint
 *     permutation of K and V (exact for non-causal attention: P'V' = PV), removal
 *     of each 128-token block's mean, E4M3 quantisation of the residual only, and
 *     exact restoration of the mean inside the online softmax from the row sums;
 *   - ExpCast-FP8: probability bytes written straight from log2-domain scores,
 *     c = clip(Round(8(u+8) + 56 + beta), 0, 120), read as E4M3.
 * (paper page paper.rainbus.top, "Method steps" (1)-(4); study notes on
 * dimensionstp.github.io, sections 2-1 to 2-4.)
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; `stream`
 *     is a hipStream_t passed as void* (NULL = the default stream).
 *   - The caller owns and allocates every buffer, workspaces included. The library
 *     never allocates, frees or synchronises, and may be called concurrently on
 *     different streams with disjoint buffers. Its only state is a per-device record
 *     of the architecture check below.
 *   - bf16 tensors are bfloat16 bit patterns; "[B,H,N,d]" means contiguous
 *     row-major with d fastest.
 *   - Arguments are validated on the host before anything is enqueued; then the
 *     current device must be a gfx950 (else VC_E_UNSUPPORTED, also when no device is
 *     present). On any error nothing is launched and outputs are untouched. A launch
 *     failure is
 *     reported as VC_E_HIP; faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP work.
 *   - Supported shapes: d in {64, 128}; block == 128; N a positive multiple of
 *     128; B, H >= 1; B*H <= 65535; B*H*N*d < 2^31. Buffers must be 16-byte aligned.
 *   - NaN or infinite inputs are not supported: outputs are then unspecified, but
 *     every kernel still terminates.
 */
#ifndef VC_H
#define VC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vc_status;
enum {
  VC_OK = 0,
  VC_E_NULLPTR = 1,     /* a required pointer is NULL */
  VC_E_SHAPE = 2,       /* B, H, N, d or block outside the supported set */
  VC_E_PARAM = 3,       /* cluster count, iteration count, beta or flags invalid */
  VC_E_WORKSPACE = 4,   /* workspace smaller than the *_workspace_bytes query */
  VC_E_UNSUPPORTED = 5, /* no gfx950 device current, or a misaligned buffer */
  VC_E_HIP = 6,         /* a HIP launch failed */
  VC_E_ALIAS = 7        /* an output overlaps an input */
};

enum {
  VC_F_KSMOOTH = 1u, /* subtract the per-channel key mean over all N tokens */
  VC_F_VSMOOTH = 2u, /* block-mean removal of V' and mean restoration */
  VC_F_EXPCAST = 4u, /* ExpCast-FP8 probability bytes (else exp2 then cast) */
  VC_F_E5M2 = 8u,    /* with VC_F_EXPCAST: the bytes are E5M2 (4 codes per octave) */
  VC_F_HADAMARD = 16u, /* quantiser: rotate Q and K~' rows by the Hadamard matrix first */
  VC_F_MXFP4 = 32u     /* 4-bit (MXFP4) value residual: vc_quantize writes it, vc_attention reads it */
};

/* Static description of a status code (host function, never NULL). */
const char* vc_status_string(vc_status s);

/* ------------------------------------------------------------------------
 * Exactness of the sums. The k-means re-rank and pair decision, the centroid, block-mean
 * and key-mean sums are sums of bf16 values (and of squared differences of bf16 values)
 * carried as binary64 pairs hi + lo: every term enters hi through an error-free addition
 * (TwoSum; squares through the FMA-based TwoProduct) and the rounding error goes to lo.
 * The readings they implement (exact argmin, exact means rounded once) hold whenever lo's
 * own additions are exact. In terms of vc_exponent_span below -- E(X) the largest exponent
 * and q(X) the lowest significand bit over the nonzero elements of a (b,h), s(X) = E(X) -
 * q(X) -- sufficient conditions per (b,h) are:
 *   - sums of n elements of X are exact when s(X) <= 103 - 2 ceil(log2 n) (every error
 *     sent to lo is a multiple of 2^q(X) of at most 2^-53 of a partial sum below
 *     n 2^(E(X)+1), and there are at most 2n of them). vc_quantize: the key mean needs
 *     s(K) <= 103 - 2 ceil(log2 N) (69 at N = 70 400; of the rotated keys when RoPE tables
 *     are given), the block means s(V) <= 89. vc_cluster, vc_cluster_balanced,
 *     vc_cluster_incremental: the member sums need s(V) <= 103 - 2 ceil(log2 N).
 *   - the squared distances sum_c (v_c - c_c)^2 (d terms) of the k-means ranking are
 *     exact when the span of V together with the bf16-rounded centroids the assignment
 *     reads (vc_exponent_span kind 2) is at most 50 - log2 d, i.e. 43 for d = 128 and 44 for
 *     d = 64 (each difference is a multiple of 2^q below 2^(E+2), each square a pair of
 *     multiples of 2^(2q), and the 2d errors sent to lo stay below 2^(2q+53)); with size
 *     penalties, each nonzero
 *     b_k = fl32(lambda n_k) must also lie in [2^(2q+23), 2^(2E+12)] (q, E of that union).
 *     The binary32 error bound that proves most labels without them assumes every nonzero
 *     |v| and |c| in [2^-56, 2^56) (no overflow or underflow in the products and norms):
 *     E <= 55 and q >= -56. With iters > 1 the centroids an assignment reads are the
 *     previous update's; run one iteration per call to check each.
 * Outside these conditions the kernels still terminate and each pair is within about
 * n^2 2^-104 (relative to the sum of the terms' magnitudes) of the exact value: a label can
 * then differ from the exact argmin only where the two best exact squared distances differ
 * by less than about 2^-88 of their size, and a mean only where its exact value lies that
 * close to a rounding boundary. Measured on the Wan-shaped benchmark step (all 40 heads): V
 * spans up to 42, K up to 32, V with the bf16 centroids of either assignment up to 42 --
 * inside every condition. The oracle is exact for every finite input.
 * ------------------------------------------------------------------------ */

/* ------------------------------------------------------------------------
 * vc_exponent_span -- the exponent range of a tensor per (batch, head), for the
 * conditions above.
 *
 *   X     device, [B,H,rows,d] contiguous; kind 0: bf16 bit patterns, kind 1: binary32,
 *         kind 2: binary32 read as the bf16 value it rounds to (nearest even), as the
 *         k-means assignment reads centroids. 2-byte (kind 0) or 4-byte aligned.
 *   out   device int32 [B,H,2], 4-byte aligned: out[2 bh] = E = the largest
 *         floor(log2 |x|), out[2 bh + 1] = q = the smallest exponent of a lowest set
 *         significand bit (every element is an integer multiple of 2^q), both over the
 *         nonzero finite elements of (b,h); an all-zero (b,h) gives (INT32_MIN, INT32_MAX).
 *         The span of a union is max(E) - min(q) of the parts.
 *   B, H, rows, d >= 1 with B*H <= 65535 and B*H*rows*d < 2^31; X and out must not overlap.
 * Deterministic (maxima and minima). Errors: VC_E_NULLPTR, VC_E_PARAM (kind), VC_E_SHAPE,
 * VC_E_UNSUPPORTED (alignment, no gfx950), VC_E_ALIAS, VC_E_HIP.
 * ------------------------------------------------------------------------ */
vc_status vc_exponent_span(const void* X, int kind, int B, int H, int rows, int d, int32_t* out, void* stream);

/* ABI version of this header (bumped on any incompatible change). */
int vc_abi_version(void);
#define VC_ABI_VERSION 2

/* ------------------------------------------------------------------------
 * vc_cluster -- online k-means on value tokens (paper page, method step (1)):
 * labels z per (batch, head), pi = argsort(z), warm-started centroids.
 *
 * Reading taken: Lloyd iterations (assign to the nearest bfloat16-rounded
 * centroid by squared Euclidean distance, exact, ties to the lowest index; then
 * centroid = binary32 rounding of the exact member mean; an empty cluster keeps
 * its centroid). `iters` >= 1 assign/update rounds. Cold start first sets
 * C_k = V[floor((2k+1)N/(2K))].
 *
 *   V          bf16 [B,H,N,d]                      input
 *   K          clusters per head, 1 <= K <= min(N, vc_max_clusters()) (8192: the label
 *              histogram of a token chunk lives in LDS); else VC_E_PARAM
 *   iters      1 <= iters <= 1000, else VC_E_PARAM
 *   centroids  float [B,H,K,d]  in: warm-start state (ignored when cold_start),
 *                               out: centroids after the last update
 *   labels     int32 [B,H,N]    out: labels of the last assignment
 *   perm       int32 [B,H,N]    out: stable argsort of labels (ties by token index)
 *   workspace  >= vc_cluster_workspace_bytes(B,H,N,d,K) bytes of device memory
 *
 * Scores: the assignment kernel ranks clusters from bf16 matrix-core dot products
 * (exact products; accumulation error measured far inside the binary32 bound the
 * test uses), keeps a rigorous per-distance error bound, and re-ranks every token whose
 * best candidate is not separated from the rest by the bounds on squared distances summed
 * as binary64 pairs, so labels equal the exact argmin whenever those pairs are exact (the
 * "Exactness" conditions above; vc_exponent_span checks them).
 * ------------------------------------------------------------------------ */
int vc_max_clusters(void); /* 8192: the largest K vc_cluster, vc_cluster_balanced and vc_cluster_incremental accept */
size_t vc_cluster_workspace_bytes(int B, int H, int N, int d, int K);
vc_status vc_cluster(const void* V, int B, int H, int N, int d, int K, int iters, int cold_start,
                     float* centroids, int32_t* labels, int32_t* perm,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vc_cluster_balanced -- vc_cluster with size-penalised assignment, a cheap form of
 * the balanced clustering the paper page's ablation measures (better error, but a
 * grouping cost its authors would not pay; balancing is on its weakness list).
 *
 * Every assignment minimises ||v - bf16(C_k)||^2 + b_k with b_k = fl32(lambda * n_k)
 * (one binary32 product), exactly, ties to the lowest index; n_k is the size of
 * cluster k after the previous assignment, taken from `counts` for the first
 * iteration. The update step is vc_cluster's. lambda = 0 gives vc_cluster's result.
 * A lambda near or above the typical gap between a token's two nearest distances
 * makes sizes oscillate between iterations (clusters can empty); a useful range is
 * a small fraction of (mean squared distance) / (N/K).
 *
 *   lambda     finite, >= 0 (else VC_E_PARAM); distance units per member
 *   counts     int32 [B,H,K]  in: sizes for the first assignment (zeros: plain
 *                             first iteration; a previous call's output: warm
 *                             start), out: sizes after the last assignment
 *   other arguments as for vc_cluster; counts must not overlap any other buffer
 *   (VC_E_ALIAS) and must be 16-byte aligned (VC_E_UNSUPPORTED)
 *
 * Exactness as for vc_cluster: the certainty bound also covers the rounding of the
 * penalised norms, and re-ranked distances are compared as the exact pair of (squared
 * distance + b_k), normalised.
 * ------------------------------------------------------------------------ */
vc_status vc_cluster_balanced(const void* V, int B, int H, int N, int d, int K, int iters, int cold_start,
                              float lambda, int32_t* counts, float* centroids, int32_t* labels, int32_t* perm,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vc_cluster_incremental -- one cross-step incremental centroid update (the paper
 * page's weakness list: clustering runs per denoising step and per head and leaves the
 * redundancy between steps unused; update centroids incrementally across steps).
 *
 * Every cluster carries a decayed member mass M_k beside its centroid. With the members
 * n_k of cluster k under the labels (re-assigned first when `assign` != 0: nearest
 * bf16(C_k), as vc_cluster assigns; else the given labels, read-only, a label outside
 * [0,K) read as 0), S_k the binary64 rounding of their exact value sum, and A = decay *
 * M_k (binary64):
 *   C_k = nearest binary32 of (A * C_k + S_k) / (A + n_k), the product, the sum and the
 *         denominator rounded in binary64 one operation at a time;
 *   M_k = fl32(A + n_k); an empty cluster keeps C_k and gets M_k = fl32(A).
 * decay 0 is one Lloyd update (with assign: one vc_cluster iteration, bit for bit);
 * decay 1 pools every step so far. perm = stable argsort of the labels.
 *
 *   decay      in [0, 1] (else VC_E_PARAM)
 *   centroids  float [B,H,K,d] in/out;  mass float [B,H,K] in/out (zeros: no history)
 *   labels     int32 [B,H,N]  out with assign, else in;  perm int32 [B,H,N] out
 *   workspace  >= vc_cluster_workspace_bytes(B,H,N,d,K)
 * Other arguments, exactness and errors as vc_cluster; no buffer may overlap another.
 * ------------------------------------------------------------------------ */
vc_status vc_cluster_incremental(const void* V, int B, int H, int N, int d, int K, float decay, int assign,
                                 float* centroids, float* mass, int32_t* labels, int32_t* perm,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vc_cluster_cost -- the k-means objective of the current values under a kept
 * clustering, a drift statistic for refreshing the permutation early (the paper
 * page's weakness list: the reused permutation loses accuracy when the layout
 * drifts; detect the drift and re-cluster).
 *
 *   V          bf16 [B,H,N,d]    current values
 *   centroids  float [B,H,K,d]   as vc_cluster left them; labels int32 [B,H,N] in [0,K)
 *   cost       double [B,H] out  (1/N) sum_t ||V_t - bf16(C_{z_t})||^2 (the assignment
 *                                distance), binary64 sums (relative error ~1e-13); a label
 *                                outside [0,K) is read as 0
 *   workspace  >= vc_cluster_cost_workspace_bytes(B,H,N,d); cost must be 8-byte aligned
 * ------------------------------------------------------------------------ */
size_t vc_cluster_cost_workspace_bytes(int B, int H, int N, int d);
vc_status vc_cluster_cost(const void* V, const float* centroids, const int32_t* labels, int B, int H, int N, int d,
                          int K, double* cost, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vc_quantize -- fused quantiser (paper page, method step (2); study notes 2-2).
 *
 *   Q, K, V    bf16 [B,H,N,d]
 *   perm       int32 [B,H,N], or NULL for the identity (plain FP8 path)
 *   block      must be 128
 *   flags      VC_F_KSMOOTH | VC_F_VSMOOTH | VC_F_HADAMARD | VC_F_MXFP4 (VC_F_EXPCAST ignored)
 * Outputs (all written on success):
 *   Qq   uint8 [B,H,N,d]           E4M3 codes of Q, original token order
 *   sQ   float [B,H,N/128]         Q block scale times fl32(log2(e)/sqrt(d))
 *   Kq   uint8 [B,H,N,d]           codes of K~' = (K - kbar)[perm], row i = token perm[i]
 *   sK   float [B,H,N/128]         K' block scales
 *   Vq   uint8 [B,H,N/128,d,128]   BLOCK-TRANSPOSED residual codes:
 *                                  Vq[b,h,j,c,t] = code of R[128j+t, c], R = V[perm] - mu
 *   sV   float [B,H,d]             per-channel residual scale (over all N tokens)
 *   mu   bf16 [B,H,N/128,d]        block means of V' (zero when !VC_F_VSMOOTH); may be NULL
 *   mu_scaled float [B,H,N/128,d]  fl32(mu / sV); may be NULL
 *   mu_pack  bf16, vc_mu_pack_size(B,H,N,d) bytes: mu_scaled in the operand layout that
 *            vc_attention consumes, [B,H,ceil(N/1024),d/32,2,64,8]: for chunk c of 8 key
 *            blocks, 32-channel block b, operand t, lane l and element s (key block 8c+s),
 *            always of channel 32b + (l mod 32): t = 0 holds bf16(mu_scaled) in all lanes;
 *            t = 1 holds bf16(mu_scaled - bf16(mu_scaled)) in lanes 0..31 and zero in
 *            lanes 32..63; key blocks past N/128 are zero. May be NULL.
 * Arithmetic: block and channel scales are fl32(amax/448) with codes
 * e4m3(fl32(x * fl32(448/amax))) (round to nearest even); amax = 0 gives scale 1
 * and zero codes; a nonzero amax below 448 / FLT_MAX (about 1.3e-36) overflows 448/amax,
 * and that block's or channel's codes are then unspecified. kbar = fl32(exact mean),
 * mu = bf16(exact block mean), on the subnormal grids where the means are that small.
 * VC_F_MXFP4 (the 4-bit residual of the pages' workstation path, as OCP MXFP4): the
 * residual R gets E2M1 codes with one E8M0 scale per group of 32 keys of a channel, the
 * scale being the smallest 2^e with max|R| <= 6 * 2^e (no clipping; 2^0 for an all-zero
 * group), codes the nearest E2M1 value of R / 2^e (ties to even mantissa, +0 for zero).
 * Group g of half q of a block holds keys 64q + 16g + {0..15} and 64q + 32 + 16g + {0..15}
 * (the 32 elements one lane of the block-scaled MFMA holds). Vq then holds, per block j
 * at byte offset 128 d j of the head: codes [c][64 bytes] -- key t of half q = t>>6 is
 * nibble p = 16((t&63)>>5) + (t&15) of group g = (t>>4)&1, at byte 32q + 16g + p/2,
 * low nibble first -- followed by scales [c][4] (E8M0 bytes, index 2q + g) at byte 64 d;
 * the rest of the block's 128 d bytes is unused. sV = 1 and mu_scaled = mu.
 * VC_F_HADAMARD (the rotation that the pages' fused preprocessing carries): every Q row
 * and every K~' row is multiplied by the unnormalised Sylvester Hadamard matrix H_d
 * before its block is quantised, evaluated as the fast Walsh-Hadamard transform in
 * binary32 (stages h = 1, 2, ..., d/2 in that order; pair (i, i+h) -> (a+b, a-b)); the
 * factor 1/d of (Q H)(K H)^T = d Q K^T is folded exactly into sQ (times 2^-log2(d)).
 * workspace >= vc_quantize_workspace_bytes(B,H,N,d,block).
 * ------------------------------------------------------------------------ */
size_t vc_quantize_workspace_bytes(int B, int H, int N, int d, int block);
size_t vc_mu_pack_size(int B, int H, int N, int d); /* bytes of mu_pack (0 if the shape is invalid) */
vc_status vc_quantize(const void* Q, const void* K, const void* V, const int32_t* perm,
                      int B, int H, int N, int d, int block, uint32_t flags,
                      uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK, uint8_t* Vq, float* sV,
                      void* mu, float* mu_scaled, void* mu_pack, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vc_quantize_noalloc -- vc_quantize for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and outputs, with no workspace argument. Its scratch is a
 * file-scope device array of VC_QUANTIZE_NOALLOC_SCRATCH_BYTES (64 MiB) that every device
 * the library runs on holds until the process ends; the call itself allocates nothing.
 *
 *   a shape whose vc_quantize_workspace_bytes exceeds VC_QUANTIZE_NOALLOC_SCRATCH_BYTES is
 *   rejected with VC_E_WORKSPACE before anything is launched (B*H*(N/128)*d up to about
 *   3.05 M elements, 22 bytes each; B=1, H=40, N=70,400, d=128 needs 59.1 MiB and fits);
 *   every call on one device shares that device's array, which keeps the last call's
 *   contents (nothing in it needs clearing: each call writes all it reads): calls that
 *   overlap in time on one device, on any streams, race and must be serialised by the
 *   caller.
 * Other arguments, outputs and errors as vc_quantize.
 * ------------------------------------------------------------------------ */
#define VC_QUANTIZE_NOALLOC_SCRATCH_BYTES (64u << 20)
vc_status vc_quantize_noalloc(const void* Q, const void* K, const void* V, const int32_t* perm,
                              int B, int H, int N, int d, int block, uint32_t flags,
                              uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK, uint8_t* Vq, float* sV,
                              void* mu, float* mu_scaled, void* mu_pack, void* stream);

/* ------------------------------------------------------------------------
 * vc_quantize_rope -- vc_quantize with rotary position embedding applied to Q and K
 * first (the pages' fused preprocessing absorbs RoPE into the quantiser).
 *
 *   rope_cos, rope_sin  float [N, d/2], shared by all (b,h): the angle of channel pair i
 *                       of token t (original order) -- any 1-D or multi-axis RoPE
 *                       expressed as per-token angles. Both required (VC_E_NULLPTR).
 * Each token's interleaved pairs (x_2i, x_2i+1) become
 *   (fl32(fl32(x_2i c) - fl32(x_2i+1 s)), fl32(fl32(x_2i s) + fl32(x_2i+1 c))),
 * rounded to bf16 (the tensor an unfused chain would hand to the quantiser), and the
 * rest is vc_quantize on the rotated Q and K (key mean over the rotated keys; a key's
 * angles are those of its original position, whatever the permutation). V is not
 * rotated. Other arguments, outputs and errors as vc_quantize.
 * ------------------------------------------------------------------------ */
vc_status vc_quantize_rope(const void* Q, const void* K, const void* V, const int32_t* perm,
                           const float* rope_cos, const float* rope_sin,
                           int B, int H, int N, int d, int block, uint32_t flags,
                           uint8_t* Qq, float* sQ, uint8_t* Kq, float* sK, uint8_t* Vq, float* sV,
                           void* mu, float* mu_scaled, void* mu_pack, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * vc_attention -- non-causal attention over the quantised tensors (paper page,
 * method steps (3) and (4); online-softmax prerequisite).
 *
 * For each query row i and every 128-key block j in ascending order:
 *   S = Qq_i . Kq_j^T on FP8 matrix cores (binary32 accumulation),
 *   sigma = fl32(sQ[i/128] * sK[j]),  m' = max(m, fl32(sigma * max S)),
 *   VC_F_EXPCAST: c = clamp(rne(fma(S, 8 sigma, fl32(fl32(120 + beta) - 8 m'))), 0, 120),
 *                 read as E4M3 (code 120 = 2^8 at u = 0)
 *   VC_F_EXPCAST | VC_F_E5M2 (ExpCast carried to E5M2, a direction the paper page's
 *                 future work names): c = clamp(rne(fma(S, 4 sigma,
 *                 fl32(fl32(120 + beta) - 4 m'))), 0, 120), read as E5M2 (code 120 =
 *                 2^15 at u = 0); the minimax offset for this format is beta = -0.17
 *   otherwise:    c = e4m3(256 * exp2(fl32(sigma S) - m')),
 *   r = row sum of the probabilities, l = 2^(m - m') l + r,
 *   A = 2^(m - m') A + c . Vq_j + r * mu_scaled_j   (mu term only if mu_pack != NULL),
 * and finally O_i = bf16(sV * A / l), rows in original token order. The r * mu term is
 * accumulated once per 8 key blocks from the bf16 hi/lo mu_pack operand (relative
 * error ~2^-16 of that term).
 *
 *   O      bf16 [B,H,N,d] output; must not overlap any input
 *   beta   finite, any sign; the pages use -0.35 (E4M3). Codes are clamped to [0, 120]
 *          for every beta (the per-byte clamp runs whenever fl32(120 + beta) > 120 or
 *          |m'| >= 2^16; below that no code can exceed 120)
 * Scores: every S is one v_mfma_f32_32x32x64_f8f6f4 per 64 channels (for d = 128 the
 * second takes the first's result as its accumulator); the matrix core sums products in
 * groups of 8 slots truncated 13 bits below each group's largest exponent and combines
 * groups with 24-bit alignment, so S is not always fl32 of the exact dot product. The
 * bytes are bit-exact functions of these S (see vc_debug_mfma_f8).
 *   flags  VC_F_EXPCAST selects ExpCast, VC_F_E5M2 its E5M2 variant (VC_E_PARAM without
 *          VC_F_EXPCAST); VC_F_KSMOOTH / VC_F_VSMOOTH are ignored, other bits VC_E_PARAM
 * ------------------------------------------------------------------------ */
vc_status vc_attention(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                       const uint8_t* Vq, const float* sV, const void* mu_pack,
                       int B, int H, int N, int d, int block, float beta, uint32_t flags,
                       void* O, void* stream);

/* Same computation, additionally writing the probability bytes that key block
 * `dump_block` received from every query: codes uint8 [B,H,N,128] (key order of
 * the block). Test support for in-kernel byte parity. */
vc_status vc_attention_dump(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                            const uint8_t* Vq, const float* sV, const void* mu_pack,
                            int B, int H, int N, int d, int block, float beta, uint32_t flags,
                            void* O, int dump_block, uint8_t* codes, void* stream);

/* ExpCast as a plain elementwise function (paper page, method step (4)): codes[i] =
 * clamp(rne(fma(acc[i], scale8[i], bias[i])), 0, 120), formed by the attention kernel's
 * own byte sequence (the inline helpers its hot loop calls): one binary32 FMA, then
 * v_cvt_pk_u8_f32 packing four bytes per dword (round half to even, saturation to
 * [0, 255]), then the packed per-byte min with 120 -- the kernel's clamped path.
 * All arrays have n elements (0 <= n <= 2^34; n = 0 is a no-op). Test support. */
vc_status vc_debug_expcast(const float* acc, const float* scale8, const float* bias, uint8_t* codes,
                           size_t n, void* stream);

/* The same without the per-byte min: the kernel's unclamped path, which it takes when no
 * byte can exceed 120 (fl32(120 + beta) <= 120 and |m'| < 2^16). Equal to
 * vc_debug_expcast whenever every fma(acc, scale8, bias) < 120.5; beyond that the bytes
 * saturate at 255 instead of 120. Test support. */
vc_status vc_debug_expcast_unclamped(const float* acc, const float* scale8, const float* bias, uint8_t* codes,
                                     size_t n, void* stream);

/* The FP8 matrix-core instruction of the attention kernel (v_mfma_f32_32x32x64_f8f6f4), one
 * 32x32x64 tile per call element: D[t] = C[t] + A[t] B[t]^T with A, B uint8 E4M3 codes
 * [ntiles][32][64] (row-major, the 64 products of an output run along the last axis) and C,
 * D float [ntiles][32][32] row-major, in the operand layout the attention kernel uses.
 * 0 <= ntiles <= 2^20; D must not overlap A, B or C (VC_E_ALIAS). Test support: it exposes
 * the score precision the kernel decides its ExpCast bytes in. */
vc_status vc_debug_mfma_f8(const uint8_t* A, const uint8_t* B, const float* C, float* D, int ntiles, void* stream);

/* Measurement support: `grid` work-groups of 4 waves each run `iters` rounds of four
 * independent v_mfma_f32_32x32x64_f8f6f4 (the attention kernel's instruction) on register
 * operands, fixed (random_bits = 0) or per-lane pseudo-random E4M3 patterns; the host times
 * it to get the sustained FP8 matrix-core rate: FLOPs = grid * 4 * iters * 4 * 131072.
 * out: float [grid * 256] scratch written by the kernel (device). */
vc_status vc_debug_mfma_peak(int grid, int iters, int random_bits, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VC_H */
