// vc_attention.hip -- VC-Attention forward for gfx950 (MI355X).
//
// Paper page (paper.rainbus.top), method steps (3) and (4); study notes 2-3, 2-4;
// online-softmax prerequisite. Non-causal; every query sees all keys.
//
// Work decomposition: one work-group = 4 waves = 128 query rows of one (b,h), 32 rows
// per wave, two work-groups per CU (the kernel below documents the per-block steps).
// Design notes for gfx950, all measured on the device:
//   - a wave issues at most one VALU instruction every ~9 cycles, two waves on a SIMD
//     reach ~4 cycles, so every SIMD keeps two waves that both carry softmax work;
//   - an FP8 MFMA blocks the SIMD's VALU issue for most of its duration; the 32x32x64
//     shape does twice the work of 16x16x128 for ~1.4x the blocking, so it is used for
//     S, PV and the row sums;
//   - K and V tiles are copied global -> LDS with buffer_load ... lds (scalar-addressed,
//     no per-lane address arithmetic) into a two-stage buffer; tile j+1 lands while
//     tile j is consumed, with one barrier per tile.
#include <type_traits>

#include "vc_device.h"

namespace vc {

constexpr int kWaves = 4;                 // waves per work-group (32 query rows each); two per CU
constexpr int kAThreads = 64 * kWaves;
constexpr int kQB = kWaves / 4;           // 128-row query blocks per work-group

// lanes l and l^32 hold the same query: combine them with one v_permlane32_swap
__device__ __forceinline__ float lane_max2(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_sum2(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS swizzles (16-byte chunk index XOR). gfx950 serves a wave's ds_read_b128 in four
// passes of 16 lanes, pass = (lane/16) xor parity(lane bits 2, 3), i.e. four interleaved
// lane quads; a pass is conflict-free when its 16 lanes hit distinct 16-byte slots modulo
// 256 bytes (64 banks). The XOR patterns below satisfy that for every fragment read.
// K tile rows are D bytes; the pattern uses row bits 1..3 (d = 128) or 2..3 (d = 64),
// which the per-MFMA key offsets (+16, +64, +80 rows) leave untouched, so a lane's K
// fragments sit at one base plus immediates. V tile rows are 128 bytes; the pattern uses
// row bits 1..3, untouched by the +32*db row offset.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * D + ((chunk ^ k_swz<D>(row)) << 4);
}
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }
// MXFP4 code rows are 64 bytes (4 chunks); row bits 2..3 keep every fragment read
// conflict-free under the same pass model, and the +32-row d-block offset leaves them alone
__device__ __forceinline__ int mx_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int v_off(int row, int chunk) { return row * 128 + ((chunk ^ v_swz(row)) << 4); }

__device__ __forceinline__ v8i ld_frag(const uint8_t* p0, const uint8_t* p1) {
  uint4 a = *reinterpret_cast<const uint4*>(p0);
  uint4 b = *reinterpret_cast<const uint4*>(p1);
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 16-byte global -> LDS copy (global_load_lds_dwordx4): lane L of the wave writes
// LDS[base + 16 L]. The builtin exists only for the device pass; seen by the host pass
// it silently drops the kernel's launch stub, so the host never compiles the call.
__device__ __forceinline__ void g2lds16(const void* src, lds_void* dst_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst_wave_base, 16, 0, 0);
#endif
}

// Buffer resource for a wave-uniform base pointer (forced into SGPRs with readfirstlane,
// so copies need no per-lane descriptor) and a record limit in bytes: an offset past the
// limit reads zeros instead of faulting. The host pass only sees a placeholder type.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#else
struct rsrc_t { int w[4]; };
#endif
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int nbytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, nbytes, 0x00020000);
#else
  (void)base; (void)nbytes;
  return rsrc_t{};
#endif
}
// Read-only data with a wave-uniform address, through the constant address space: the
// load becomes a scalar s_load, which never waits behind the tile copies the way a
// vector load's vmcnt would.
typedef const __attribute__((address_space(4))) float* const_f32_ptr;
__device__ __forceinline__ float uniform_load(const float* p, int i) {
  return ((const_f32_ptr)p)[i];
}
// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane L of the wave writes
// LDS[base + 16 L] from the resource at voff + soff. Device pass only (see g2lds16).
__device__ __forceinline__ void buf2lds16(rsrc_t r, int voff, int soff, lds_void* dst_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst_wave_base, 16, voff, soff, 0, 0);
#else
  (void)r; (void)voff; (void)soff; (void)dst_wave_base;
#endif
}

// Work-group barrier without a memory fence: LDS tiles are only written by the
// asynchronous copies, whose completion the loop waits for explicitly, and every wave
// has consumed the fragments it read before it arrives (the MFMAs that use them are
// issued first). The clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// vmcnt(0) only (expcnt 7, lgkmcnt 15 left open), through the builtin so that the compiler's
// own wait tracking knows the copies are complete
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// One work-group = 4 waves = 128 query rows of one (b,h), 32 rows per wave; two
// work-groups per CU, so every SIMD runs two waves whose vector-ALU work interleaves with
// the other's matrix-core work. The key loop walks the 128-key blocks in ascending order
// (ExpCast bytes depend on the running maximum, so the loop is never split or reordered).
//
// Per key block, per wave (32 queries = one 32x32 MFMA column block):
//   S^T (keys x queries) = K_j Q^T with v_mfma_f32_32x32x64_f8f6f4: MFMA kb (0..3) per
//   64-wide d half takes the key rows kappa(kb, r) = 64(kb>>1) + 32((r>>2)&1) + 16(kb&1)
//   + 4(r>>3) + (r&3), so accumulator element i of lane l holds key 64(kb>>1) + 32(l/32)
//   + 16(kb&1) + i of query l%32: exactly byte 16(kb&1)+i of the PV B operand that lane
//   supplies for the 64-key half kb>>1. The probability bytes never leave the lane.
//   Row max: 64 values in-lane, then lanes l and l^32 combine (v_permlane32_swap).
//   Row sum of the ExpCast bytes: two MFMAs with an all-ones A operand.
//   O^T (d x queries) += V_j^T P^T with the same instruction (K = 64 keys per half).
//   Mean restoration: O^T[c][q] += r_q mu~_j[c], accumulated on the matrix core once
//   per 8 key blocks (bf16 hi/lo split, v_mfma_f32_32x32x16_bf16).
// PM selects the probability bytes: 0 exp-then-cast (E4M3), 1 ExpCast E4M3 (8 codes per
// octave, code 120 = 2^8), 2 ExpCast E5M2 (4 codes per octave, code 120 = 2^15; the PV and
// row-sum MFMAs read their B operand as BF8).
// MX selects the 4-bit value residual (MXFP4): V tiles hold E2M1 codes [channel][64 bytes]
// in the block-scaled MFMA's operand order plus one E8M0 scale per channel and 32-key group.
template <int D, int PM, bool RESTORE, bool DUMP, bool MX>
__global__ __launch_bounds__(kAThreads, 8 / kWaves) void attn_fwd(const uint8_t* __restrict__ Qq, const float* __restrict__ sQ,
                                                         const uint8_t* __restrict__ Kq, const float* __restrict__ sK,
                                                         const uint8_t* __restrict__ Vq, const float* __restrict__ sV,
                                                         const uint16_t* __restrict__ mu_pack, int N, int total,
                                                         float C0, uint16_t* __restrict__ O, int dump_block,
                                                         uint8_t* __restrict__ dump) {
  constexpr bool EXPCAST = PM != 0;
  constexpr int PFMT = PM == 2 ? 1 : 0;         // MFMA operand format of the bytes: FP8 or BF8
  constexpr float SLOPE = PM == 2 ? 4.0f : 8.0f; // ExpCast codes per octave
  constexpr int TILE = kBlock * D;              // bytes per K (or V) tile
  constexpr int NCH = TILE / 16;                // 16-byte chunks per tile
  constexpr int PW = NCH / kAThreads;           // chunks per thread per tile (4 or 2)
  constexpr int NDB = D / 32;                   // 32-channel blocks of O
  constexpr int NDH = D / 64;                   // 64-wide d halves of the S contraction
  constexpr int CPR = D / 16;                   // 16-byte chunks per K row
  constexpr int PACK = NDB * 2 * 64 * 16;       // mean operand of one chunk of 8 key blocks
  constexpr int RLOG = kWaves * 8 * 32 * 8;     // waves x slots x queries x (r, m')
  // Two stages each of K and V as separate arrays, always indexed by compile-time stage
  // numbers (the loop below is unrolled by two): the compiler can then prove that fragment
  // reads of one stage never alias the asynchronous copies into the other, and inserts no
  // wait for those copies before the reads.
  __shared__ __attribute__((aligned(16))) uint8_t kst0[TILE], kst1[TILE], vst0[TILE], vst1[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t packs[RESTORE ? PACK : 16];
  // the row-sum log has an array of its own: written with ordinary LDS stores, it must not
  // look to the compiler as if it could alias the mean operand's asynchronous copies
  __shared__ __attribute__((aligned(16))) float2 rlog_all[RESTORE ? RLOG / 8 : 2];
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  const int nb = N / kBlock;
  // work-group indices are uniform; readfirstlane makes that visible to the compiler so
  // address arithmetic on them stays scalar
  const int nwg = (nb + kQB - 1) / kQB;         // work-groups per (b,h)
  const int logical = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, total));
  const int bh = logical / nwg, wgq = logical % nwg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  // query block of this wave; a missing last block (N/128 not a multiple of the blocks per
  // work-group) is computed on the last real block and not stored
  const int qb_raw = kQB * wgq + wave / 4;
  const bool store = qb_raw < nb;
  const int qb = min(qb_raw, nb - 1);
  const int q = qb * kBlock + (wave & 3) * 32 + r32;  // this lane's query row

  const uint8_t* Kh = Kq + (size_t)bh * N * D;
  const uint8_t* Vh = Vq + (size_t)bh * N * D;
  const int nchunk = (nb + 7) / 8;
  const float sq = sQ[(size_t)bh * nb + qb];
  const float* sKh = sK + (size_t)bh * nb;  // per-tile scales, read with scalar loads

  // ---- Q fragments (B operand of S^T): query row, bytes [64 dh + 32 h, +32)
  v8i qf[NDH];
  for (int dh = 0; dh < NDH; dh++) {
    const uint4* src = reinterpret_cast<const uint4*>(Qq + ((size_t)bh * N + q) * D + 64 * dh + 32 * h);
    uint4 a = src[0], b = src[1];
    qf[dh][0] = a.x; qf[dh][1] = a.y; qf[dh][2] = a.z; qf[dh][3] = a.w;
    qf[dh][4] = b.x; qf[dh][5] = b.y; qf[dh][6] = b.z; qf[dh][7] = b.w;
  }
  // Row sums on the matrix core: read as the B operand of v_mfma_f32_16x16x128_f8f6f4, a
  // PV operand pf[kh] gives column c = l%16 the key bytes of query c (lane groups 0, 2)
  // and of query c+16 (lane groups 1, 3). The A operand row m selects one of the two:
  // it is E4M3 1.0 (0x38) where ((m>>2)&1) equals the lane group's query half and zero
  // elsewhere, so output rows 4(l/16)..+3, which lane l receives, all hold the row sum of
  // query l%32.
  v8i sel;
  {
    const int on = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 0x38383838 : 0;
    for (int k = 0; k < 8; k++) sel[k] = on;
  }

  // ---- tile copies (buffer -> LDS, lane L of a wave fills LDS chunk base+L). The source of
  // each chunk is chosen so that LDS ends up in the swizzled layout; a thread's chunks i > 0
  // sit 32 K rows (64 for d = 64) further on, which the swizzles ignore, so one per-lane
  // offset serves all of them and the rest goes into the scalar offset.
  const rsrc_t krs = make_rsrc(Kh, N * D), vrs = make_rsrc(Vh, N * D);
  int ksrc, vsrc;
  {
    const int P = wave * 64 + lane;
    const int row = P / CPR, phys = P % CPR;
    ksrc = row * D + 16 * (phys ^ k_swz<D>(row));
    if (MX) {  // code rows are 64 bytes: 4 chunks, XOR pattern (row >> 2) & 3
      const int vrow = P >> 2, vphys = P & 3;
      vsrc = vrow * 64 + 16 * (vphys ^ mx_swz(vrow));
    } else {
      const int vrow = P >> 3, vphys = P & 7;
      vsrc = vrow * 128 + 16 * (vphys ^ v_swz(vrow));
    }
  }
  auto issue_k = [&](int j, auto st) {  // K_j into stage st (= j & 1)
    uint8_t* kd = decltype(st)::value ? kst1 : kst0;
    for (int i = 0; i < PW; i++)
      buf2lds16(krs, ksrc, j * TILE + i * kAThreads * 16, (lds_void*)(kd + (wave * 64 + kAThreads * i) * 16));
  };
  auto issue_v = [&](int j, auto st) {  // V_j into stage st (= j & 1)
    uint8_t* vd = decltype(st)::value ? vst1 : vst0;
    if (MX) {  // 64 D bytes of codes, then 4 D bytes of scales (wave 0, lanes < D/4)
      for (int i = 0; i < PW / 2; i++)
        buf2lds16(vrs, vsrc, j * TILE + i * kAThreads * 16, (lds_void*)(vd + (wave * 64 + kAThreads * i) * 16));
      if (wave == 0 && lane < D / 4) buf2lds16(vrs, lane * 16, j * TILE + 64 * D, (lds_void*)(vd + 64 * D));
    } else {
      for (int i = 0; i < PW; i++)
        buf2lds16(vrs, vsrc, j * TILE + i * kAThreads * 16, (lds_void*)(vd + (wave * 64 + kAThreads * i) * 16));
    }
  };
  // mean operand of chunk c: NDB x 2 MFMAs x 64 lanes x 16 bytes, one 1 KB piece per wave
  auto issue_pack = [&](int c) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(mu_pack) + ((size_t)bh * nchunk + c) * PACK;
    const rsrc_t r = make_rsrc(src, PACK);
    for (int piece = wave; piece < PACK / 1024; piece += kWaves)
      buf2lds16(r, lane * 16, piece * 1024, (lds_void*)(packs + piece * 1024));
  };

  // fixed per-lane fragment offsets (bytes, within a stage)
  const int krow0 = 32 * ((r32 >> 2) & 1) + 4 * (r32 >> 3) + (r32 & 3);
  int kA[NDH], kB[NDH];
  for (int dh = 0; dh < NDH; dh++) {
    kA[dh] = k_off<D>(krow0, 4 * dh + 2 * h);
    kB[dh] = k_off<D>(krow0, 4 * dh + 2 * h + 1);
  }
  const int vA0 = v_off(r32, 2 * h), vB0 = v_off(r32, 2 * h + 1);
  const int vA1 = v_off(r32, 4 + 2 * h), vB1 = v_off(r32, 4 + 2 * h + 1);
  // MXFP4: lane (r32, h) of half kh reads chunk 2 kh + h of code row r32 (+32 per d block)
  const int vM0 = r32 * 64 + 16 * ((0 + h) ^ mx_swz(r32)), vM1 = r32 * 64 + 16 * ((2 + h) ^ mx_swz(r32));

  float m = -__builtin_inff(), lsum = 0.0f;
  v16f oacc[NDB];
  for (int db = 0; db < NDB; db++)
    for (int i = 0; i < 16; i++) oacc[db][i] = 0.0f;
  v16f zero16;
  for (int i = 0; i < 16; i++) zero16[i] = 0.0f;
  const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  // Mean restoration on the matrix core: each key block's row sum r_j is logged with the
  // running max m'_j it is scaled to; once per 8 key blocks the logged sums are brought to
  // the current max, w = r_j 2^(m'_j - m'), split into bf16 hi + lo, and folded in with two
  // v_mfma_f32_32x32x16_bf16 per 32-channel block: K slots 0..7 (lanes 0-31) take
  // mu_hi x w_hi, slots 8..15 (lanes 32-63) mu_hi x w_lo, and the second MFMA mu_lo x w_hi.
  // Log layout per wave [slot][query]: 32 lanes touch 256 contiguous bytes.
  float2* const rlog = rlog_all + wave * (8 * 32);
  auto flush = [&](int nvalid, float mref) {
    float2 t[8];
    for (int k = 0; k < 8; k++) t[k] = rlog[k * 32 + r32];
    // pairs of weights: hi = bf16(w) and lo = bf16(w - hi), two per conversion; lanes of
    // the upper half supply the low parts (and zeros to the second MFMA)
    v8i w0, w1;
    for (int k2 = 0; k2 < 4; k2++) {
      f32x2 w;
      w.x = 2 * k2 < nvalid ? t[2 * k2].x * __builtin_amdgcn_exp2f(t[2 * k2].y - mref) : 0.0f;
      w.y = 2 * k2 + 1 < nvalid ? t[2 * k2 + 1].x * __builtin_amdgcn_exp2f(t[2 * k2 + 1].y - mref) : 0.0f;
      const bf16x2 hb = __builtin_convertvector(w, bf16x2);
      uint32_t hp;
      __builtin_memcpy(&hp, &hb, 4);
      const f32x2 r = {w.x - __uint_as_float(hp << 16), w.y - __uint_as_float(hp & 0xffff0000u)};
      const bf16x2 lb = __builtin_convertvector(r, bf16x2);
      uint32_t lp;
      __builtin_memcpy(&lp, &lb, 4);
      w0[k2] = (int)(h ? lp : hp);
      w1[k2] = h ? 0 : (int)hp;
    }
    bf16x8 b0, b1;
    __builtin_memcpy(&b0, &w0, 16);
    __builtin_memcpy(&b1, &w1, 16);
    for (int db = 0; db < NDB; db++) {
      bf16x8 a0, a1;
      __builtin_memcpy(&a0, packs + (db * 2 + 0) * 1024 + lane * 16, 16);
      __builtin_memcpy(&a1, packs + (db * 2 + 1) * 1024 + lane * 16, 16);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, oacc[db], 0, 0, 0);
    }
  };

  // S for key groups kb0, kb0+1 of the tile in stage `stage` (d halves accumulated)
  v16f sacc[4];
  auto s_part = [&](auto st, int kb0) {
    const uint8_t* kt = decltype(st)::value ? kst1 : kst0;
    for (int kb = kb0; kb < kb0 + 2; kb++) {
      const int ko = (64 * (kb >> 1) + 16 * (kb & 1)) * D;
      for (int dh = 0; dh < NDH; dh++) {
        const v8i a = ld_frag(kt + kA[dh] + ko, kt + kB[dh] + ko);
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[dh], dh == 0 ? zero16 : sacc[kb], 0, 0, 0, 0, 0, 0);
      }
    }
  };
  // O^T += V_j^T P^T for the 64-key half kh
  auto pv_part = [&](const uint8_t* vt, int kh, const v8i& p) {
    if (MX) {
      // A: 32 E2M1 codes in 4 dwords (keys 16h..+15 and 32+16h..+15 of the half); its E8M0
      // scale, byte 2 kh + h of the channel's four, scales exactly those 32 elements
      for (int db = 0; db < NDB; db++) {
        const uint4 f = *reinterpret_cast<const uint4*>(vt + (kh ? vM1 : vM0) + 32 * db * 64);
        v8i a;
        a[0] = f.x; a[1] = f.y; a[2] = f.z; a[3] = f.w; a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
        const int sc = vt[64 * D + 4 * (32 * db + r32) + 2 * kh + h];
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p, oacc[db], 4, PFMT, 0, sc, 0, 127);
      }
      return;
    }
    const int A0 = kh ? vA1 : vA0, B0 = kh ? vB1 : vB0;
    for (int db = 0; db < NDB; db++) {
      const int vo = 32 * db * 128;
      const v8i a = ld_frag(vt + A0 + vo, vt + B0 + vo);
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, p, oacc[db], 0, PFMT, 0, 0, 0, 0);
    }
  };

  // Pipeline: K runs one tile ahead of V. Iteration j holds K_{j+1} and V_j in LDS while
  // K_{j+2} and V_{j+1} land in the other stages; S_j was computed in iteration j-1.
  issue_k(0, S0{});
  if (nb > 1) issue_k(1, S1{});
  issue_v(0, S0{});
  if (RESTORE) issue_pack(0);
  wait_copies();
  __syncthreads();
  s_part(S0{}, 0);
  s_part(S0{}, 2);
  // iteration 0 copies K_2 into stage 0: every wave must have read K_0 from it first
  wg_barrier();

  // iteration j; P = j & 1 is a compile-time stage number
  auto iteration = [&](int j, auto P) {
    constexpr int p = decltype(P)::value;
    using Other = std::integral_constant<int, 1 - p>;
    const uint8_t* vt = p ? vst1 : vst0;  // V_j
    const float sigma = sq * uniform_load(sKh, j);
    if (j + 2 < nb) issue_k(j + 2, P);                 // replaces K_j, consumed in iteration j-1
    if (j + 1 < nb) issue_v(j + 1, Other{});           // replaces V_{j-1}
    // chunk c = j/8 replaces chunk c-1, which every wave flushed before the last barrier
    if (RESTORE && j > 1 && (j & 7) == 1) issue_pack(j >> 3);

    // ---- running max over S_j
    float mx;
    {
      float v[64];
      for (int kb = 0; kb < 4; kb++)
        for (int i = 0; i < 16; i++) v[16 * kb + i] = sacc[kb][i];
      float w[22];
      for (int i = 0; i < 21; i++) w[i] = fmaxf(fmaxf(v[3 * i], v[3 * i + 1]), v[3 * i + 2]);
      w[21] = v[63];
      float x[8];
      for (int i = 0; i < 7; i++) x[i] = fmaxf(fmaxf(w[3 * i], w[3 * i + 1]), w[3 * i + 2]);
      x[7] = w[21];
      const float y0 = fmaxf(fmaxf(x[0], x[1]), x[2]), y1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
      mx = lane_max2(fmaxf(fmaxf(y0, y1), fmaxf(x[6], x[7])));
    }
    const float mnew = sigma * mx;
    const float mp = fmaxf(m, mnew);
    const float alpha = __builtin_amdgcn_exp2f(m - mp);
    if (__ballot(alpha != 1.0f))
      for (int db = 0; db < NDB; db++) oacc[db] *= alpha;

    // ---- probability bytes per 64-key half; the PV MFMAs of a half and the next tile's
    // S MFMAs for the freed accumulators are issued as soon as the half is done, so the
    // matrix core works while the vector ALU converts the other half.
    v8i pf[2];
    float r = 0.0f;
    v4f rs;
    // ExpCast bytes (the helpers in vc_device.h): FMA, cvt_pk_u8_f32, and the per-byte min with
    // 120 only when some byte can exceed it (beta above ~0.45, or |m'| >= 2^16; uniform per wave)
    const bool fix = EXPCAST && __ballot(expcast_needs_clamp(C0, mp));
    auto bytes_half = [&](int kh) {
      if (EXPCAST) {
        // All 32 FMAs of the half first (in place: the accumulators are dead afterwards),
        // then the byte conversions with the eight packed words interleaved. Written one
        // word at a time, each conversion waits on the FMA issued just before it and on
        // the previous byte of the same word: one serial chain through the whole half.
        const float bias = C0 - SLOPE * mp;
        const float s8 = SLOPE * sigma;
        for (int kb = 2 * kh; kb < 2 * kh + 2; kb++)
          for (int i = 0; i < 16; i++) sacc[kb][i] = expcast_t(sacc[kb][i], s8, bias);
        uint32_t w[8];
        for (int k = 0; k < 8; k++) w[k] = expcast_cvt<0>(sacc[2 * kh + (k >> 2)][4 * (k & 3)], 0u);
        for (int k = 0; k < 8; k++) w[k] = expcast_cvt<1>(sacc[2 * kh + (k >> 2)][4 * (k & 3) + 1], w[k]);
        for (int k = 0; k < 8; k++) w[k] = expcast_cvt<2>(sacc[2 * kh + (k >> 2)][4 * (k & 3) + 2], w[k]);
        for (int k = 0; k < 8; k++) w[k] = expcast_cvt<3>(sacc[2 * kh + (k >> 2)][4 * (k & 3) + 3], w[k]);
        for (int k = 0; k < 8; k++) pf[kh][k] = (int)w[k];
        if (fix)
          for (int k = 0; k < 8; k++) pf[kh][k] = (int)expcast_min120((uint32_t)pf[kh][k]);
        return;
      }
      // exp-then-cast
      for (int kb = 2 * kh; kb < 2 * kh + 2; kb++)
        for (int qd = 0; qd < 4; qd++) {
          const float p0 = 256.0f * __builtin_amdgcn_exp2f(sigma * sacc[kb][4 * qd + 0] - mp);
          const float p1 = 256.0f * __builtin_amdgcn_exp2f(sigma * sacc[kb][4 * qd + 1] - mp);
          const float p2 = 256.0f * __builtin_amdgcn_exp2f(sigma * sacc[kb][4 * qd + 2] - mp);
          const float p3 = 256.0f * __builtin_amdgcn_exp2f(sigma * sacc[kb][4 * qd + 3] - mp);
          // both conversions as one opaque step right after the exponentials: written
          // with the builtins, the compiler keeps all 32 scaled values of the half live
          // until the PV operand is needed and then spills with the MXFP4 value path;
          // op_sel[3] writes the high word and keeps the low one
          uint32_t w;
          asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2\n\tv_cvt_pk_fp8_f32 %0, %3, %4 op_sel:[0,0,1]"
                       : "=&v"(w) : "v"(p0), "v"(p1), "v"(p2), "v"(p3));
          r += (p0 + p1) + (p2 + p3);
          pf[kh][4 * (kb & 1) + qd] = (int)w;
        }
    };
    bytes_half(0);
    pv_part(vt, 0, pf[0]);
    s_part(Other{}, 0);  // K_{j+1} (stale, and unused, after the last tile)
    bytes_half(1);
    if (EXPCAST) {  // row sum of the decoded bytes on the matrix core
      rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pf[0], zero4, 0, PFMT, 0, 0, 0, 0);
      rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pf[1], rs, 0, PFMT, 0, 0, 0, 0);
    }
    // the wave's last ten MFMAs have no vector work of its own to overlap: raised issue
    // priority keeps the matrix core fed from this wave while the SIMD's other wave
    // converts (0.5 % shorter launch, measured)
    __builtin_amdgcn_s_setprio(2);
    pv_part(vt, 1, pf[1]);
    s_part(Other{}, 2);
    __builtin_amdgcn_s_setprio(0);
    if (RESTORE && j > 0 && (j & 7) == 0) flush(8, mp);  // chunk j/8 - 1, scaled to the new max
    r = EXPCAST ? rs[0] : lane_sum2(r);

    lsum = __builtin_fmaf(alpha, lsum, r);
    if (RESTORE && h == 0) rlog[(j & 7) * 32 + r32] = make_float2(r, mp);
    m = mp;
    if (DUMP && j == dump_block && store) {
      uint4* dst = reinterpret_cast<uint4*>(dump + ((size_t)bh * N + q) * kBlock + 32 * h);
      dst[0] = make_uint4(pf[0][0], pf[0][1], pf[0][2], pf[0][3]);
      dst[1] = make_uint4(pf[0][4], pf[0][5], pf[0][6], pf[0][7]);
      dst[4] = make_uint4(pf[1][0], pf[1][1], pf[1][2], pf[1][3]);
      dst[5] = make_uint4(pf[1][4], pf[1][5], pf[1][6], pf[1][7]);
    }
    // copies of this iteration landed, and every wave is done with the stages they replace
    wait_copies();
    wg_barrier();
  };
  for (int j = 0; j < nb; j += 2) {
    iteration(j, S0{});
    if (j + 1 < nb) iteration(j + 1, S1{});
  }

  if (RESTORE) {
    const int clast = (nb - 1) >> 3;
    if (clast > 0 && 8 * clast + 1 >= nb) {  // a one-block last chunk was not copied in the loop
      issue_pack(clast);
      wait_copies();
      wg_barrier();
    }
    flush(nb - 8 * clast, m);
  }

  // ---- epilogue: O = bf16(sV * A / l); element i of block db is channel 32 db + 8(i/4) + 4h + i%4
  if (!store) return;
  const float il = 1.0f / lsum;
  uint16_t* orow = O + ((size_t)bh * N + q) * D;
  for (int db = 0; db < NDB; db++)
    for (int g = 0; g < 4; g++) {
      const int c = 32 * db + 8 * g + 4 * h;
      const float4 s4 = *reinterpret_cast<const float4*>(sV + (size_t)bh * D + c);
      uint32_t w0 = (uint32_t)f32_to_bf16(s4.x * oacc[db][4 * g + 0] * il) | ((uint32_t)f32_to_bf16(s4.y * oacc[db][4 * g + 1] * il) << 16);
      uint32_t w1 = (uint32_t)f32_to_bf16(s4.z * oacc[db][4 * g + 2] * il) | ((uint32_t)f32_to_bf16(s4.w * oacc[db][4 * g + 3] * il) << 16);
      *reinterpret_cast<uint2*>(orow + c) = make_uint2(w0, w1);
    }
}

// The hot loop's byte sequence on elementwise inputs, four per thread (one packed dword, as
// the kernel forms them): FMA, cvt_pk_u8_f32 into byte 0..3, then the per-byte min with 120
// when `clamp` (the kernel's rare path) -- without it, inputs must keep every FMA result
// below 120.5, as the kernel guarantees before it skips the min.
__global__ void expcast_kernel(const float* __restrict__ acc, const float* __restrict__ s8, const float* __restrict__ bias,
                               uint8_t* __restrict__ out, size_t n, int clamp) {
  const size_t i0 = 4 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  float t[4];
  for (int e = 0; e < 4; e++) t[e] = i0 + e < n ? expcast_t(acc[i0 + e], s8[i0 + e], bias[i0 + e]) : 0.0f;
  uint32_t w = expcast_cvt<0>(t[0], 0u);
  w = expcast_cvt<1>(t[1], w);
  w = expcast_cvt<2>(t[2], w);
  w = expcast_cvt<3>(t[3], w);
  if (clamp) w = expcast_min120(w);
  for (int e = 0; e < 4; e++)
    if (i0 + e < n) out[i0 + e] = (uint8_t)(w >> (8 * e));
}

template <int D, int PM, bool R, bool DU, bool MX>
static void launch_attn(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK, const uint8_t* Vq,
                        const float* sV, const uint16_t* mu, int BH, int N, float C0, uint16_t* O, int dump_block,
                        uint8_t* dump, hipStream_t st) {
  const int total = BH * ((N / kBlock + kQB - 1) / kQB);
  attn_fwd<D, PM, R, DU, MX><<<total, kAThreads, 0, st>>>(Qq, sQ, Kq, sK, Vq, sV, mu, N, total, C0, O, dump_block, dump);
}

template <int D, int PM, bool MX>
static void launch_attn_d(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK, const uint8_t* Vq,
                          const float* sV, const uint16_t* mu, int BH, int N, float C0, uint16_t* O, int dump_block,
                          uint8_t* dump, hipStream_t st) {
  if (mu) {
    if (dump) launch_attn<D, PM, true, true, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
    else launch_attn<D, PM, true, false, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
  } else {
    if (dump) launch_attn<D, PM, false, true, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
    else launch_attn<D, PM, false, false, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
  }
}

template <int D, bool MX>
static void launch_attn_pm(int pmode, const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                           const uint8_t* Vq, const float* sV, const uint16_t* mu, int BH, int N, float C0,
                           uint16_t* O, int dump_block, uint8_t* dump, hipStream_t st) {
  if (pmode == 2) launch_attn_d<D, 2, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
  else if (pmode == 1) launch_attn_d<D, 1, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
  else launch_attn_d<D, 0, MX>(Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
}

}  // namespace vc

using namespace vc;

// pmode: 0 exp-then-cast, 1 ExpCast E4M3, 2 ExpCast E5M2; mx: 4-bit (MXFP4) value residual
extern "C" int vc_launch_attention(const uint8_t* Qq, const float* sQ, const uint8_t* Kq, const float* sK,
                                   const uint8_t* Vq, const float* sV, const void* mu_pack, int B, int H, int N, int d,
                                   float beta, int pmode, int mx, uint16_t* O, int dump_block, uint8_t* dump,
                                   hipStream_t st) {
  const uint16_t* mu = (const uint16_t*)mu_pack;
  const int BH = B * H;
  const float C0 = 120.0f + beta;  // fl32(120 + beta)
  if (d == 128) {
    if (mx) launch_attn_pm<128, true>(pmode, Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
    else launch_attn_pm<128, false>(pmode, Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
  } else {
    if (mx) launch_attn_pm<64, true>(pmode, Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
    else launch_attn_pm<64, false>(pmode, Qq, sQ, Kq, sK, Vq, sV, mu, BH, N, C0, O, dump_block, dump, st);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int vc_launch_expcast(const float* acc, const float* s8, const float* bias, uint8_t* out, size_t n,
                                 int clamp, hipStream_t st) {
  if (n == 0) return 0;
  const size_t blocks = (n + 1023) / 1024;   // 256 threads x 4 elements
  expcast_kernel<<<(unsigned)blocks, 256, 0, st>>>(acc, s8, bias, out, n, clamp);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
