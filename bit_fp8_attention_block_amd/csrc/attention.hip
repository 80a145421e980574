// ExpCast FP8 attention kernel for gfx950.
//
// Method (VC-Attention write-up, "ExpCast-FP8" section; Open VC Attention
// product page, kernel paragraph): each softmax weight is written as its E4M3
// byte straight from the log-domain score with one FMA. No exponential is
// evaluated and no FP32->FP8 conversion is made. With a = 8*tau*log2(e)*sq*sk
// for the (query block, key tile) pair and the bit-aligned running row max M,
//     byte = clamp(rne(a*s_raw + (119.65 - 8*M)), 0, 255)
// is one v_fma_f32 per score and one v_cvt_pknorm_u16_f32 per two scores
// (rounding to nearest, clamping), plus a byte permute per four. The byte
// never exceeds 120 because M >= ceil(a*s_raw/8), and scores more than ~15
// binades below the max land on 0.
//
// For comparison the same kernel can instead take the path ExpCast replaces
// (weights selection OC_WEIGHTS_EXP_FP8): weight 256*2^(x - M) from v_exp_f32,
// then the hardware FP32 -> E4M3 cast (v_cvt_pk_fp8_f32), with everything else
// (max, frame scale, sums, MFMAs) unchanged.
//
// Because M is an integer, the weights of earlier tiles relative to a stale M
// differ from those relative to the new M by an exact power of two. O and L
// are kept in the frame of a reference max, and each tile's weights enter it
// through that power of two as the E8M0 scale of the PV MFMA's P operand, so
// growth of M costs no rescale of O and L; the result does not depend on the
// key-tile order (up to the underflow tail).
//
// Layout of the work (one workgroup = 256 queries of one (b, h)):
//  * S^T = K Q^T on v_mfma_f32_16x16x128_f8f6f4. Lane l then holds keys
//    16t + 4g + r (g = l/16) of query l%16 for each 16x16 output block.
//  * those bytes, 32 per lane, are used as-is as the B operand of
//    O^T = V^T P^T on the same MFMA. V was packed transposed in the
//    matching key order by the prepare step, so P never leaves registers.
//  * the row sum L is one more MFMA per 16 queries against an all-ones A
//    operand (E4M3 1.0 = 0x38), so the VALU never decodes bytes.
//  * K and V tiles (16 KiB each) stream through LDS by direct global->LDS
//    loads (global_load_lds_dwordx4). The prepare step stores them in MFMA
//    operand order, so every operand read is a contiguous, bank-conflict-
//    free ds_read_b128.
//  * row max across the 4 lanes that share a query: v_permlane16/32_swap.
//  * key tiles are visited from the middle of the key window outwards
//    (c, c-1, c+1, ... with c = (nT-1)/2; Open VC Attention product page,
//    kernel paragraph; Open-VC news, "Архитектурные оптимизации"). The
//    order is the same for every query tile of a head. Bytes are relative to
//    the running max, so the result is that of the single-pass form of the
//    method in this order.
//  * workgroups are mapped so that each XCD walks consecutive query tiles
//    of the same heads; as they share the key order, a K/V tile fetched by
//    one workgroup is found in the XCD's L2 by the others.
#include "oc_common.h"
#include "oc_kernels.h"

namespace oc {

__device__ inline v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
  // v_mfma_f32_16x16x128_f8f6f4 with A and B as OCP E4M3 (format 0), no block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The same with the B operand's values multiplied by 2^(sb - 127) (E8M0 block
// scale in byte 0 of sb, per lane, i.e. per column and 32-element K block);
// the power-of-two factor is exact.
__device__ inline v4f mfma_f8_sb(const v8i& a, const v8i& b, const v4f& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// The MFMA operand of 16-row block `blk` for this lane: 32 bytes, read as two
// contiguous 1 KiB wave accesses from an operand-ordered LDS tile
__device__ inline v8i lds_operand(const uint8_t* tile, int blk, int lane) {
  const uint4 x = *reinterpret_cast<const uint4*>(tile + ((2 * blk) * 64 + lane) * 16);
  const uint4 y = *reinterpret_cast<const uint4*>(tile + ((2 * blk + 1) * 64 + lane) * 16);
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}

// key tile visited at step s: the centre tile c, then c-1, c+1, c-2, c+2, ...,
// continuing on the longer side once the shorter one is exhausted
// (order 1: ascending, for tests)
__device__ inline int tile_at(int s, int c, int nT, int order) {
  if (order == 1) return s;
  if (s == 0) return c;
  const int left = c, right = nT - 1 - c;
  const int m = min(left, right);
  if (s <= 2 * m) {
    const int d = (s + 1) >> 1;
    return (s & 1) ? c - d : c + d;
  }
  const int extra = s - 2 * m;
  return left > right ? c - m - extra : c + m + extra;
}

// One 16 KiB tile from global memory into LDS by direct global->LDS loads,
// the LDS copy laid out as the tile is in memory. Threads 0..NT-1 take part:
// wave wv copies the contiguous 16384*64/NT bytes at wv*16384*64/NT, one KiB
// per instruction, lane l's 16 bytes landing at the wave's LDS base + 16*l.
// The base comes from M0 and the instruction's immediate offset (i KiB) is
// added to both the global and the LDS address, so a wave sets M0 once per
// tile and the loads differ only in that immediate; the global address is a
// scalar base plus the per-lane offset lane16 = 16*lane. Issuing a tile
// costs no vector instructions.
// Written as inline assembly so that the compiler does not track these loads:
// it would otherwise drain all of them (vmcnt(0)) before every LDS read and
// at every barrier, which rules out keeping a tile load in flight across an
// iteration. The caller orders them with explicit vmcnt waits and
// lds_barrier(). The s_nop covers the M0-write -> LDS-DMA hazard.
template <int NT>
__device__ inline void load_tile(uint32_t lds_dst, const uint8_t* src, uint32_t lane16, int wv) {
  constexpr int PER = 1024 / NT;   // instructions (KiB) per wave
  static_assert(PER == 2 || PER == 4, "a tile is split over 4 or 8 waves");
  const uint32_t base = (uint32_t)wv * (PER * 1024u);
  const uint32_t m0 = lds_dst + base;
  const uint8_t* g = src + base;
  if constexpr (PER == 2)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:1024"
                 :
                 : "s"(m0), "v"(lane16), "s"(g)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:3072"
                 :
                 : "s"(m0), "v"(lane16), "s"(g)
                 : "memory", "m0");
}

// byte offset in the workgroup's LDS of a pointer into it
__device__ inline uint32_t lds_offset(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Workgroup barrier that orders LDS accesses only (a full __syncthreads
// fence would also wait for every outstanding global load)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int QBW = 2;            // 16-query blocks per wave
constexpr int NWAVES = 8;         // 2 waves per SIMD: one of each group
constexpr int NTHREADS = 64 * NWAVES;
constexpr int NBUF = 4;                    // K and V tiles, four buffers each
constexpr int LDS_BYTES = 2 * NBUF * TILE_BYTES;
// V-Smooth: the tile's block means (128 bf16 = 256 B) ride with each V tile
constexpr int MU_SLOT = 256;
// 32 slots: the mean term of sixteen tiles is added at once (vsmooth_flush)
// while the means of later tiles are being loaded
constexpr int MU_NBUF = 32;
constexpr int LDS_BYTES_VS = LDS_BYTES + MU_NBUF * MU_SLOT;

// The 256 bytes of one tile's block means into an LDS slot by one wave's
// direct load of 4 bytes per lane (voff = 4*lane)
__device__ inline void load_means(uint32_t lds_dst, const uint8_t* src, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_dst), "v"(voff), "s"(src)
               : "memory", "m0");
}

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int SG_MFMA = 0x008, SG_VALU = 0x002, SG_DS_READ = 0x100;

// LDS operand read-ahead of the tile loops, in 16-row blocks: the operand of
// block kb+RA is read while the MFMAs of block kb run
constexpr int RA = 2;
// K operands of its next QK that group B reads before each barrier
constexpr int KPRE = 2;

// largest lag (binades) of the reference max of O and L behind the running max
constexpr float FRAME_DRIFT = 64.0f;

// c += A B with B's values times 2^(sb - 127), as inline assembly (`one` is a
// register holding 127, the A operand's unit scale). The PV accumulation uses
// this form: through the builtin, the register allocator handled its
// accumulators badly enough to spill (256 VGPRs and about 130 spilled,
// against 235 and none written out). The compiler does not look inside the
// statement, so it inserts no wait states for it: every access to c or b by
// other instructions next to it is separated by hand, with pfence before the
// first such MFMA of a tile (after the VALU writes of P) and ofence before
// VALU or another MFMA type touches O. A CPU test scans the compiled kernels
// for any access that escapes these fences.
__device__ __forceinline__ void mfma_f8_sb_acc(v4f& c, const v8i& a, const v8i& b, int one, int sb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(c)
               : "v"(a), "v"(b), "v"(one), "v"(sb));
}
// 4 wait states between the VALU writes of the P operand and the MFMAs that
// read it (the hardware asks for 2)
__device__ __forceinline__ void pfence(v8i (&P)[QBW]) {
  asm volatile("s_nop 3" : "+v"(P[0]), "+v"(P[1]));
}
// 24 wait states: more than an 8-pass XDL result needs before VALU reads or
// overwrites it, or an MFMA of another type accumulates into it
__device__ __forceinline__ void ofence(v4f (&O)[QBW][8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(O[0][0]), "+v"(O[0][1]), "+v"(O[0][2]), "+v"(O[0][3]), "+v"(O[0][4]), "+v"(O[0][5]),
                 "+v"(O[0][6]), "+v"(O[0][7]), "+v"(O[1][0]), "+v"(O[1][1]), "+v"(O[1][2]), "+v"(O[1][3]),
                 "+v"(O[1][4]), "+v"(O[1][5]), "+v"(O[1][6]), "+v"(O[1][7]));
}

// S^T = K Q^T for one 128-key tile and the wave's 32 queries, with the K
// operands read RA blocks ahead, so the LDS latency hides behind 2*RA MFMAs
// instead of stalling every pair. The first NPRE (0 or >= RA) operands were
// read by the caller (pre).
template <int NPRE = 0>
__device__ __forceinline__ void qk_tile(const uint8_t* kt, const v8i (&qop)[QBW], v4f (&S)[QBW][8], int lane,
                                        const v8i* pre = nullptr) {
  static_assert(NPRE == 0 || (NPRE >= RA && NPRE <= 8), "read-ahead");
  v8i kop[8];
#pragma unroll
  for (int kb = 0; kb < (NPRE ? NPRE : RA); ++kb) kop[kb] = NPRE ? pre[kb] : lds_operand(kt, kb, lane);
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    if (kb + RA < 8 && kb + RA >= NPRE) kop[kb + RA] = lds_operand(kt, kb + RA, lane);
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) S[qb][kb] = mfma_f8(kop[kb], qop[qb], v4f{0.f, 0.f, 0.f, 0.f});
  }
  if (!NPRE) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * RA, 0);
#pragma unroll
  for (int kb = 0; kb < 8 - RA; ++kb) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, QBW, 0);
    if (kb + RA >= NPRE) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, RA * QBW, 0);
}

// O^T += V^T P^T and (ROWSUM) L += 1 * P^T for one tile, with the same
// read-ahead. With PRE the first RA operands were read by the caller (pre).
// ASM false issues the same MFMA through the compiler builtin: the code-dump
// variant of the kernel (a parity aid that spills registers) uses it, so that
// the compiler sees the accumulators and separates its spill code from them.
template <bool ROWSUM = true, bool PRE = false, bool ASM = true>
__device__ __forceinline__ void pv_tile(const uint8_t* vt, v8i (&P)[QBW], const int (&sb)[QBW], int one,
                                        v4f (&O)[QBW][8], v4f (&L)[QBW], int lane, const v8i& ones,
                                        const v8i* pre = nullptr) {
  pfence(P);
  v8i vop[8];
#pragma unroll
  for (int n = 0; n < RA; ++n) vop[n] = PRE ? pre[n] : lds_operand(vt, n, lane);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    if (n + RA < 8) vop[n + RA] = lds_operand(vt, n + RA, lane);
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      if (ASM) mfma_f8_sb_acc(O[qb][n], vop[n], P[qb], one, sb[qb]);
      else O[qb][n] = mfma_f8_sb(vop[n], P[qb], O[qb][n], sb[qb]);
    }
  }
  if (ROWSUM) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) L[qb] = mfma_f8_sb(ones, P[qb], L[qb], sb[qb]);
  }
  if (!PRE) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * RA, 0);
#pragma unroll
  for (int n = 0; n < 8 - RA; ++n) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, QBW, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, ROWSUM ? (RA + 1) * QBW : RA * QBW, 0);
}

// V-Smooth restore. The output gains sum_t l_t * mu_t, with l_t the row sum of
// tile t's weights and mu_t its bf16 block means (times inv = 448/amax of the
// head's smoothed V; the output is multiplied by sv = 1/inv at the end). This
// is a contraction over tiles, so it runs on the MFMA, sixteen tiles at a
// time: O^T[d][q] += sum_k mu_k[d] * (inv * l_k[q]).
//
// vsmooth_tile: the row sum of tile t goes into row k = t%16 of the
// accumulator C (C[k][q] += l_t[q]). The row-sum MFMA takes the all-ones A
// operand with E8M0 scale 1 on the lanes of row k (asel = 127 where
// l16 == k) and 2^-127 on the others (asel = 0), so the other rows gain at
// most 2^-127 * l_t, far below the output's rounding.
__device__ __forceinline__ void vsmooth_tile(const v8i (&P)[QBW], const int (&sb)[QBW], v4f (&C)[QBW], int asel,
                                             const v8i& ones) {
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb)
    C[qb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P[qb], C[qb], 0, 0, 0, asel, 0, sb[qb]);
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// vsmooth_flush: adds the batch of steps last - last%16 .. last and clears C.
// C is in the layout of the bf16 16x16x16 MFMA's B operand (lane (q, g) holds
// rows 4g..4g+3 of query q). inv * C is split into a truncated bf16 high part
// and a bf16 low part (truncated too; error below 2^-16 of the value), and
// each goes through one MFMA per 16 channels with the means as A: lane
// (i, g) holds mu[16n + i] of the batch's steps 4g..4g+3, read as 2-byte
// values from their LDS slots. Slots of steps past `last` hold older means
// or zeros, against rows of C that hold no row sum. L gains the column sums
// of C (over the 4 lanes of each query). C reaches 2^83 in the frame (16
// tiles x 128 keys x 256 x 2^64), so where inv exceeds 2^40 (amax of the
// smoothed V below about 4e-10) the excess power of two goes onto the means
// instead, exactly (through fp32); inv * C stays below 2^124.
__device__ __forceinline__ void vsmooth_flush(const uint8_t* mubuf, int last, float inv, v4f (&O)[QBW][8],
                                              v4f (&L)[QBW], v4f (&C)[QBW], int g, int l16) {
  const int s0 = last & ~15;
  const uint16_t* mp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    mp[i] = reinterpret_cast<const uint16_t*>(mubuf + ((s0 + 4 * g + i) & (MU_NBUF - 1)) * MU_SLOT) + l16;
  int ash = 0;   // uniform: inv is the head's
  if (inv > 0x1p40f) {
    ash = (int)(__float_as_uint(inv) >> 23) - 127 - 40;   // inv is positive and normal here
    inv = __builtin_ldexpf(inv, -ash);
  }
  v4s A[8];
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) A[n][i] = (short)mp[i][16 * n];
  if (ash > 0) {
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        A[n][i] = (short)(__float_as_uint(__builtin_ldexpf(__uint_as_float((uint32_t)(uint16_t)A[n][i] << 16), ash)) >> 16);
  }
  v4s Bh[QBW], Bl[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    float cs = (C[qb][0] + C[qb][1]) + (C[qb][2] + C[qb][3]);
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    L[qb] += cs;
    uint32_t u[4], w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float c = C[qb][r] * inv;
      u[r] = __float_as_uint(c);
      w[r] = __float_as_uint(c - __uint_as_float(u[r] & 0xFFFF0000u));
    }
    const uint32_t h01 = __builtin_amdgcn_perm(u[1], u[0], 0x07060302u), h23 = __builtin_amdgcn_perm(u[3], u[2], 0x07060302u);
    const uint32_t l01 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u), l23 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
    Bh[qb] = __builtin_bit_cast(v4s, v2u{h01, h23});
    Bl[qb] = __builtin_bit_cast(v4s, v2u{l01, l23});
    C[qb] = v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      O[qb][n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[n], Bh[qb], O[qb][n], 0, 0, 0);
      O[qb][n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[n], Bl[qb], O[qb][n], 0, 0, 0);
    }
}

// NaN-propagating maximum: scores are finite or -inf, and unlike fmaxf this
// needs no canonicalisation of MFMA results, so it maps to one v_maximum3_f32
// per two new operands
__device__ __forceinline__ float fmax_p(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// max of the 32 scores a lane holds for one 16-query block: two chains of
// three-operand maxima (17 instructions, dependent depth 9)
__device__ __forceinline__ float lane_max32(const v4f (&Sc)[8]) {
  float c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const v4f* x = Sc + 4 * h;
    float m = fmax_p(fmax_p(x[0][0], x[0][1]), x[0][2]);
    m = fmax_p(fmax_p(m, x[0][3]), x[1][0]);
    m = fmax_p(fmax_p(m, x[1][1]), x[1][2]);
    m = fmax_p(fmax_p(m, x[1][3]), x[2][0]);
    m = fmax_p(fmax_p(m, x[2][1]), x[2][2]);
    m = fmax_p(fmax_p(m, x[2][3]), x[3][0]);
    m = fmax_p(fmax_p(m, x[3][1]), x[3][2]);
    c[h] = fmax_p(m, x[3][3]);
  }
  return fmax_p(c[0], c[1]);
}

// Four scores of one query -> four E4M3 bytes (low byte first).
// ExpCast: byte = clamp(rne(a*s + b), 0, 255), with a = 8*tau*log2(e)*sq*sk and
// b = 119.65 - 8*M. The FMA is taken with a and b divided by 65535 and the
// result converted two scores at a time by the unorm16 conversion, which
// rounds clamp(y', 0, 1)*65535 to the nearest integer without an intermediate
// rounding of the product (checked on every value of a 16.7M-value sweep);
// one byte permute then packs the four low bytes. With the running max raised
// first, a*s + b <= 119.65, so the low byte is the whole code. Against one
// convert per score this saves a quarter of the conversions; the divided
// operands move about 1 byte in 10^5 by one code.
__device__ __forceinline__ uint32_t bytes_expcast(const v4f& sc, float a, float b) {
  const auto lo = __builtin_amdgcn_cvt_pknorm_u16(__builtin_fmaf(sc[0], a, b), __builtin_fmaf(sc[1], a, b));
  const auto hi = __builtin_amdgcn_cvt_pknorm_u16(__builtin_fmaf(sc[2], a, b), __builtin_fmaf(sc[3], a, b));
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x06040200u);
}
// Exp path: weight 2^(a8*s + b8) with a8 = a/8 and b8 = 8 - M, i.e. 256*2^(x - M)
// (at most 256, so the cast never saturates; -inf gives 0), cast to E4M3 with
// round-to-nearest-even by the hardware.
__device__ __forceinline__ uint32_t bytes_exp_fp8(float e0, float e1, float e2, float e3) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false) & 0xFFFFu;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, (int)lo, true);
}
__device__ __forceinline__ uint32_t bytes_exp(const v4f& sc, float a8, float b8) {
  return bytes_exp_fp8(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[0], a8, b8)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(sc[1], a8, b8)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2], a8, b8)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(sc[3], a8, b8)));
}

// The 4 lanes of a query are l, l^16, l^32, l^48: the same position in the
// four 16-lane rows of the wave. Exchanges of whole rows between two
// registers (v_permlane16_swap: rows 1, 3 of the first with rows 0, 2 of the
// second; v_permlane32_swap: rows 2, 3 of the first with rows 0, 1 of the
// second) let both 16-query blocks share each step.
__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __uint_as_float(x); }

// Max over the 4 lanes of each query of x0 (block 0) and x1 (block 1): the
// result holds block 0's maxima in rows 0 and 2 and block 1's in rows 1 and 3.
__device__ __forceinline__ float row_max_pair(float x0, float x1) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(f2u(x0), f2u(x1), false, false);
  const float c = fmax_p(u2f(s16[0]), u2f(s16[1]));   // rows: b0 of rows 0-1, b1 of rows 0-1, b0 of 2-3, b1 of 2-3
  const auto s32 = __builtin_amdgcn_permlane32_swap(f2u(c), f2u(c), false, false);
  return fmax_p(u2f(s32[0]), u2f(s32[1]));
}

// A value held per block as above (block = row parity) -> both blocks' values
// in every lane.
__device__ __forceinline__ void spread_pair(float v, float& v0, float& v1) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v0 = u2f(s16[0]);
  v1 = u2f(s16[1]);
}

// ExpCast for one tile and the wave's two 16-query blocks: raise the running
// bit-aligned max (and with it the power-of-two scale that brings the tile's
// bytes into the frame of O and L), then one FMA per score and one
// conversion per two scores give the E4M3 bytes. The running max Mv is kept per block by row parity (rows 0, 2:
// block 0; rows 1, 3: block 1), so that the max, the ceiling, the growth
// test and the FMA addend take one instruction for both blocks. aq8 is
// 8*tau*log2(e)*sq/8 for the wave's 32 queries, which share one 128-query
// scale block.
template <bool DUMP, bool EXPP>
__device__ __forceinline__ void expcast_tile(v4f (&S)[QBW][8], v8i (&P)[QBW], float (&b)[QBW], float aq8, float skj, float& Mv,
                                             float& Mr, int (&sb)[QBW], v4f (&O)[QBW][8], v4f (&L)[QBW],
                                             v4f (&C)[QBW], int j, bool masked, const AttnArgs& a, int g,
                                             const int (&dslot)[QBW]) {
  if (masked) {
    // keys beyond S in the last (ragged) tile take no part in max or sums.
    // The empty asm makes lim opaque, so that the 32 compares stay in this
    // rarely taken branch instead of being hoisted out of the tile loop as
    // 32 loop-invariant lane masks (64 SGPRs, which then spill).
    int lim = a.S - j * KTILE - 4 * g;   // this lane's key 16kb + r is dead when 16kb + r >= lim
    if (!DUMP) asm volatile("" : "+v"(lim));
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool dead = 16 * kb + r >= lim;
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb)
          if (dead) S[qb][kb][r] = -__builtin_inff();
      }
  }
  static_assert(QBW == 2, "the per-block exchanges assume two 16-query blocks per wave");
  const float aqs8 = aq8 * skj;   // a/8, a = 8*tau*log2(e)*sq*sk
  const float mv = row_max_pair(lane_max32(S[0]), lane_max32(S[1]));
  const float Mn = fmax_p(Mv, __builtin_ceilf(aqs8 * mv));
  if (__builtin_amdgcn_ballot_w64(Mn > Mv) != 0) {
    // O and L stay in the frame of a reference max Mr: the bytes of this tile
    // weigh 2^(Mn - Mr) there, a factor the PV and row-sum MFMAs apply as the
    // E8M0 scale of their P operand. O and L are rescaled (exactly, by a
    // power of two) only where the frame would fall more than FRAME_DRIFT
    // binades behind. The running max starts at -inf and the frame at 0, so
    // on the first tile the frame moves to the tile's max unless that lies in
    // [0, FRAME_DRIFT] (O and L are still zero then); from there on
    // Mr <= Mv.
    float e = Mn - Mr;
    if (__builtin_amdgcn_ballot_w64(e > FRAME_DRIFT || e < 0.0f) != 0) {
      ofence(O);
      const bool re = e > FRAME_DRIFT || e < 0.0f;
      float d0, d1;   // exponent change of each block (<= 0)
      spread_pair(re ? -e : 0.0f, d0, d1);
      const int d[QBW] = {(int)d0, (int)d1};
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[qb][n][r] = __builtin_ldexpf(O[qb][n][r], d[qb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) L[qb][r] = __builtin_ldexpf(L[qb][r], d[qb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) C[qb][r] = __builtin_ldexpf(C[qb][r], d[qb]);   // V-Smooth row sums not yet added
      }
      Mr = re ? Mn : Mr;
      e = re ? 0.0f : e;
    }
    float e0, e1;
    spread_pair(e, e0, e1);
    sb[0] = 127 + (int)e0;
    sb[1] = 127 + (int)e1;
    Mv = Mn;
    // the FMA's addend per block, in every lane, follows the running max
    // (ExpCast: a and b over 65535, for bytes_expcast's unorm16 conversion)
    spread_pair(EXPP ? 8.0f - Mn : __builtin_fmaf(-8.0f / 65535.0f, Mn, EXPCAST_C / 65535.0f), b[0], b[1]);
  }
  // a/65535 is the same in every lane of the wave: it goes to an SGPR, so the
  // 64 FMAs of a tile read two VGPRs each instead of three. (The empty
  // statement hides that the value is uniform, which would let the compiler
  // drop the readfirstlane and keep it in a VGPR.)
  float aqs_v = aqs8 * (8.0f / 65535.0f);
  asm volatile("" : "+v"(aqs_v));
  const float aqs = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, aqs_v)));
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      if (EXPP)
        P[qb][kb] = (int)bytes_exp(S[qb][kb], aqs8, b[qb]);
      else
        P[qb][kb] = (int)bytes_expcast(S[qb][kb], aqs, b[qb]);
    }
  if (DUMP) {
    float mq[QBW];
    spread_pair(Mn, mq[0], mq[1]);
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      const int slot = dslot[qb];
      if (slot >= 0) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = j * KTILE + 16 * kb + 4 * g + r;
            if (key < a.S) {
              const int64_t at = (int64_t)slot * a.S + key;
              if (a.dump_codes != nullptr) a.dump_codes[at] = (uint8_t)((uint32_t)P[qb][kb] >> (8 * r));
              if (a.dump_scores != nullptr) a.dump_scores[at] = S[qb][kb][r];
            }
          }
        if (g == 0 && a.dump_m != nullptr) a.dump_m[(int64_t)slot * a.nT + j] = (int32_t)mq[qb];
      }
    }
  }
}

// Row-list slot of a query row in the dump (the first index i with
// rows[i] == row), or -1. The search only ever narrows [lo, hi), so it ends
// within log2(n) + 1 steps and stays inside the list whatever it holds.
__device__ inline int dump_slot(const AttnArgs& a, int row) {
  int lo = 0, hi = a.n_dump;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a.dump_rows[mid] < row) lo = mid + 1;
    else hi = mid;
  }
  return (lo < a.n_dump && a.dump_rows[lo] == row) ? lo : -1;
}

// the two parts of the tile loop (see the kernel)
template <bool V>
struct bool_tag {
  static constexpr bool value = V;
};

// End of an iteration: wait for the loads this wave issued one iteration ago
// (a tile is 4 loads per thread, plus one 1 KiB load on wave 0 for V-Smooth
// block means), keeping this iteration's in flight; `all` drains everything.
__device__ __forceinline__ void wait_loads(bool all, bool ld_k, bool ld_v, bool ld_x) {
  if (all) __builtin_amdgcn_s_waitcnt(0x0F70);                               // vmcnt(0)
  else if (ld_k && ld_v) {
    if (ld_x) __builtin_amdgcn_s_waitcnt(0x0F79);                             // vmcnt(9)
    else __builtin_amdgcn_s_waitcnt(0x0F78);                                  // vmcnt(8)
  } else if (ld_k || ld_v) {
    if (ld_x) __builtin_amdgcn_s_waitcnt(0x0F75);                             // vmcnt(5)
    else __builtin_amdgcn_s_waitcnt(0x0F74);                                  // vmcnt(4)
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// One workgroup = 256 queries of one (b, h): 8 waves of 32 queries. Waves
// 0-3 (group A) and 4-7 (group B) share the SIMDs pairwise and run the
// same tile loop half an iteration apart, so that on every SIMD one wave
// issues MFMAs while the other runs the VALU part:
//   group A, iteration s:  loads, ExpCast(s) | PV(s), QK(s+1)
// (group A reads its first PV operands before the ExpCast, so that its MFMA
// phase starts without an LDS wait)
//   group B, iteration s:  QK(s), PV(s-1)    | ExpCast(s)
// (group B reads the first operands of QK(s+1) and PV(s) after its ExpCast,
// before the barrier; the two groups run separate copies of the loop, so
// group B holds no scores across it and has the registers for them)
// Group B starts its MFMAs right after the barrier, at raised priority, so
// the partner wave's MFMAs do not interleave with them and delay B's ExpCast.
// Only group A issues the tile loads (issuing the 32 KiB of one iteration
// takes several hundred cycles, which would otherwise hold back B's MFMAs).
// Iteration s reads K tiles s and s+1 and V tiles s-1 and s. The loads issued
// in iteration s (K s+3, V s+2) may stay in flight until the end of
// iteration s+1, which hides L2 misses; so K and V get four LDS buffers each
// (128 KiB).
// Work items are (b, h, 256-query tile), numbered b-major; XCD x (the
// workgroups i with i % 8 == x) owns the contiguous range [x*per, x*per + n_x),
// so the workgroups one XCD runs at a time share K/V tiles in its L2. Under
// full load the XCDs do not run at one speed (their mean workgroup times
// differ by up to 5%), and a fixed split ends with the slowest. So a range's
// first s0 items go by workgroup index, and the rest are claimed at run time:
// a claiming workgroup first takes the next item of its own XCD's range, and
// once that is used up, the next item of the range with the most items left.
// ctr[0..7] count the claims made on each range, ctr[8] the claiming
// workgroups that are done claiming; the last of them sets all nine back to
// zero, once no claim can follow.
// Every item is run exactly once: claim k on range x returns k once, and a
// workgroup gives up only once it has seen every range used up (counters only
// grow within a launch, so a count at or past a range's size stays there);
// with at least as many claiming workgroups as claimed items, none is left.
__device__ inline int claim_item(uint32_t* ctr, int nwork, int per, int s0, int n_claim) {
  const int x = blockIdx.x & 7;
  // claimable items of range y; claims compare unsigned, so that no counter
  // value can give an item outside the range
  auto range_left = [&](int y) { return (uint32_t)max(min(per, nwork - y * per) - s0, 0); };
  int item = -1;
  uint32_t i = __hip_atomic_fetch_add(&ctr[x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (i < range_left(x)) item = x * per + s0 + (int)i;
  uint32_t used_up = 1u << x;
  while (item < 0) {
    int best = -1;
    uint32_t most = 0;
    for (int k = 1; k < 8; ++k) {
      const int y = (x + k) & 7;
      if ((used_up >> y) & 1u) continue;
      const uint32_t c = __hip_atomic_load(&ctr[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t n = range_left(y);
      if (c < n && n - c > most) { most = n - c; best = y; }
    }
    if (best < 0) break;
    i = __hip_atomic_fetch_add(&ctr[best], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < range_left(best)) item = best * per + s0 + (int)i;
    else used_up |= 1u << best;
  }
  const uint32_t done = __hip_atomic_fetch_add(&ctr[8], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (done == (uint32_t)n_claim - 1u) {
    for (int y = 0; y < 9; ++y) __hip_atomic_store(&ctr[y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return item;
}

template <bool REPAIR, bool DUMP, bool EXPP, bool VSMOOTH>
__global__ __launch_bounds__(NTHREADS) void attn_kernel(AttnArgs a) {
  __shared__ int claimed;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t* const kbuf = smem;
  uint8_t* const vbuf = smem + NBUF * TILE_BYTES;
  uint8_t* const mubuf = smem + 2 * NBUF * TILE_BYTES;   // V-Smooth only

  int b, h, qt;
  if (DUMP) {
    b = a.dump_b; h = a.dump_h; qt = blockIdx.x;
  } else {
    const int nwork = a.B * a.H * a.nQT;
    const int per = (nwork + 7) >> 3;
    const int j = blockIdx.x >> 3;
    int w;
    if (j < a.sched_s0) {
      w = (blockIdx.x & 7) * per + j;
      if (w >= nwork) return;
    } else {
      if (threadIdx.x == 0) claimed = claim_item(a.sched, nwork, per, a.sched_s0, a.sched_n_claim);
      __syncthreads();
      w = claimed;
      if (w < 0) return;
    }
    qt = w % a.nQT;
    const int bh_ = w / a.nQT;
    h = bh_ % a.H;
    b = bh_ / a.H;
  }
  const int bh = b * a.H + h;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool group_b = wv >= NWAVES / 2;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  // LDS offsets of the K, V and block-mean buffers, and the per-lane offsets
  // of the direct loads
  const uint32_t kofs = lds_offset(kbuf), vofs = lds_offset(vbuf), mofs = lds_offset(mubuf);
  const uint32_t voff = 16u * lane, voff_mu = 4u * lane;
  const int q0 = qt * BQ + wv * QBW * 16;
  const int qrow0 = q0 + l16;
  const int nT = a.nT;
  int dslot[QBW] = {-1, -1};   // dump slots of this lane's two query rows
  if (DUMP) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb)
      if (qrow0 + 16 * qb < a.S) dslot[qb] = dump_slot(a, qrow0 + 16 * qb);
  }

  // Q^T operands stay in registers for the whole loop
  v8i qop[QBW];
  float aq[QBW];   // equal: the wave's 32 queries lie in one 128-query scale block
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const uint8_t* p = a.qhat + ((int64_t)bh * a.s_pad_q + q0 + 16 * qb + l16) * HEAD_DIM + 32 * g;
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint4 y = *reinterpret_cast<const uint4*>(p + 16);
    qop[qb][0] = x.x; qop[qb][1] = x.y; qop[qb][2] = x.z; qop[qb][3] = x.w;
    qop[qb][4] = y.x; qop[qb][5] = y.y; qop[qb][6] = y.z; qop[qb][7] = y.w;
    aq[qb] = a.c8 * a.sq[(int64_t)bh * a.nQB + ((q0 + 16 * qb) >> 7)];
  }

  // the all-ones operand of the row-sum MFMAs (E4M3 1.0 = 0x38), made opaque
  // so that it stays in registers instead of being rebuilt every tile
  v8i ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;
  asm volatile("" : "+v"(ones));
  v4f O[QBW][8], L[QBW], S[QBW][8];
  v8i P[QBW];
  float Mv = -__builtin_inff();    // running max per block by row parity (see expcast_tile)
  float bq[QBW] = {0.0f, 0.0f};    // the ExpCast FMA's addend for Mv (set when Mv first grows)
  v4f C[QBW];                      // V-Smooth: row sums of the current batch of sixteen tiles
  float Mr = 0.0f;                 // reference max of O and L, same layout
  int sb[QBW] = {127, 127};        // E8M0 scale of the P operand: 2^(M - Mr)
  int one = 127;                   // the V operand's unit scale, in a register
  asm volatile("" : "+v"(one));
  const float aq8 = aq[0] * 0.125f;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    L[qb] = v4f{0.f, 0.f, 0.f, 0.f};
    C[qb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 8; ++n) O[qb][n] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  const uint8_t* kg = a.kpack + (int64_t)bh * nT * TILE_BYTES;
  const uint8_t* vg = a.vpack + (int64_t)bh * nT * TILE_BYTES;
  // per-tile K scales through the scalar cache: a vector load here would sit
  // behind the tile loads in the vector memory counter
  const __attribute__((address_space(4))) float* skp =
      (const __attribute__((address_space(4))) float*)(a.sk + (int64_t)bh * nT);
  const int centre = (nT - 1) >> 1;
  const int last_masked = (a.S & (KTILE - 1)) ? nT - 1 : -1;

  const auto kt_ptr = [&](int step) { return kg + (int64_t)tile_at(step, centre, nT, a.order) * TILE_BYTES; };
  const auto vt_ptr = [&](int step) { return vg + (int64_t)tile_at(step, centre, nT, a.order) * TILE_BYTES; };
  // prologue: K steps 0..2 and V steps 0..1
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (i < nT) load_tile<NTHREADS>(kofs + i * TILE_BYTES, kt_ptr(i), voff, wvs);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (i < nT) load_tile<NTHREADS>(vofs + i * TILE_BYTES, vt_ptr(i), voff, wvs);
  const auto mu_of = [&](int tile) {
    return reinterpret_cast<const uint8_t*>(a.vmu + ((int64_t)bh * nT + tile) * HEAD_DIM);
  };
  const auto mu_ptr = [&](int step) { return mu_of(tile_at(step, centre, nT, a.order)); };
  const float vinv = VSMOOTH ? a.sv[2 * bh + 1] : 0.0f;
  if (VSMOOTH) {
    // slots of steps never loaded are read by the last flush of a short
    // sequence (against rows of C without a row sum): zero, not stale LDS
    static_assert(MU_NBUF * MU_SLOT == 16 * NTHREADS, "one 16-byte store per thread");
    *reinterpret_cast<uint4*>(mubuf + 16 * tid) = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  if (VSMOOTH && wv == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (i < nT) load_means(mofs + i * MU_SLOT, mu_ptr(i), voff_mu);
  }
  __builtin_amdgcn_s_waitcnt(0);   // this wave's chunks are in LDS
  __syncthreads();
  if (!group_b) qk_tile(kbuf, qop, S, lane);
  // first operands read ahead of their MFMAs, so those start without an LDS
  // wait. pre: group A, V operands of its PV, read before its ExpCast;
  // group B, K operands of its next QK. bpre: group B, V operands of its next
  // PV. Group B reads both before the barrier that ends an iteration.
  v8i pre[KPRE > RA ? KPRE : RA];
  v8i bpre[RA];
  // group A carries the key tiles of steps s, s+1 and s+2 (the ExpCast's
  // scale, the V load) from one iteration to the next and works out only
  // that of step s+3 (the K load)
  int ta0 = tile_at(0, centre, nT, a.order), ta1 = tile_at(1, centre, nT, a.order);
  int ta2 = tile_at(2, centre, nT, a.order);

  // One iteration of the tile loop. Before the last three steps (TAIL
  // false) every tile load is issued, so the load flags are constants.
  const auto iteration = [&](int s, auto tail, auto grp) {
    constexpr bool TAIL = decltype(tail)::value;
    constexpr bool GB = decltype(grp)::value;   // group B
    const int j = GB ? tile_at(s, centre, nT, a.order) : ta0;
    const int b0 = s & (NBUF - 1), b1 = (s + 1) & (NBUF - 1), bm1 = (s - 1) & (NBUF - 1);
    const bool ld_k = !TAIL || s + 3 < nT, ld_v = !TAIL || s + 2 < nT;
    const int t3 = (ld_k && !GB) ? tile_at(s + 3, centre, nT, a.order) : 0;
    if (!GB) {
      // V tile s is in LDS since the last barrier: its first operands arrive
      // while the ExpCast below runs, so the PV MFMAs start without waiting
#pragma unroll
      for (int i = 0; i < RA; ++i) pre[i] = lds_operand(vbuf + b0 * TILE_BYTES, i, lane);
    }
    // (group A is waves 0-3, threads 0-255)
    if (ld_k && !GB) load_tile<NTHREADS / 2>(kofs + ((s + 3) & (NBUF - 1)) * TILE_BYTES, kg + (int64_t)t3 * TILE_BYTES, voff, wvs);
    if (ld_v && !GB) load_tile<NTHREADS / 2>(vofs + ((s + 2) & (NBUF - 1)) * TILE_BYTES, vg + (int64_t)ta2 * TILE_BYTES, voff, wvs);
    // V-Smooth: one more 1 KiB load on wave 0, the block means of tile s+2
    const bool ld_mu = VSMOOTH && ld_v && wv == 0;
    if (ld_mu) load_means(mofs + ((s + 2) & (MU_NBUF - 1)) * MU_SLOT, mu_of(ta2), voff_mu);
    const float skj = skp[j];
    if (!GB) {
      expcast_tile<DUMP, EXPP>(S, P, bq, aq8, skj, Mv, Mr, sb, O, L, C, j, j == last_masked, a, g, dslot);
      if (VSMOOTH) vsmooth_tile(P, sb, C, l16 == (s & 15) ? 127 : 0, ones);
      pv_tile<!VSMOOTH, true, !DUMP>(vbuf + b0 * TILE_BYTES, P, sb, one, O, L, lane, ones, pre);
      if (VSMOOTH && ((s & 15) == 15 || s + 1 == nT)) {
        ofence(O);
        vsmooth_flush(mubuf, s, vinv, O, L, C, g, l16);
        ofence(O);
      }
      if (s + 1 < nT) qk_tile(kbuf + b1 * TILE_BYTES, qop, S, lane);
      ta0 = ta1;
      ta1 = ta2;
      ta2 = t3;
    } else {
      __builtin_amdgcn_s_setprio(2);
      qk_tile<KPRE>(kbuf + b0 * TILE_BYTES, qop, S, lane, pre);
      if (s > 0) pv_tile<!VSMOOTH, true, !DUMP>(vbuf + bm1 * TILE_BYTES, P, sb, one, O, L, lane, ones, bpre);
      // the batch that ended with tile s-1 (before ExpCast(s) may re-anchor)
      if (VSMOOTH && s > 0 && ((s - 1) & 15) == 15) {
        ofence(O);
        vsmooth_flush(mubuf, s - 1, vinv, O, L, C, g, l16);
        ofence(O);
      }
      __builtin_amdgcn_s_setprio(0);
      expcast_tile<DUMP, EXPP>(S, P, bq, aq8, skj, Mv, Mr, sb, O, L, C, j, j == last_masked, a, g, dslot);
      if (VSMOOTH) vsmooth_tile(P, sb, C, l16 == (s & 15) ? 127 : 0, ones);
      // K step s+1 and V step s have been in LDS since the last barrier: the
      // first operands of the next QK and PV arrive before the next one
      if (s + 1 < nT) {
#pragma unroll
        for (int i = 0; i < KPRE; ++i) pre[i] = lds_operand(kbuf + b1 * TILE_BYTES, i, lane);
      }
#pragma unroll
      for (int i = 0; i < RA; ++i) bpre[i] = lds_operand(vbuf + b0 * TILE_BYTES, i, lane);
    }
    // group A waits for the loads it issued one iteration ago (a tile is 4
    // loads per thread, plus one for the block means on wave 0 with
    // V-Smooth); this iteration's stay in flight. The code dump's stores also
    // count, so that path drains everything.
    wait_loads(DUMP || GB, ld_k, ld_v, ld_mu);
    lds_barrier();
  };
  // one loop per group, so that each keeps only its own values live across
  // the back edge (group B holds no scores there, group A no weights)
  int s = 0;
  if (group_b) {
#pragma unroll
    for (int i = 0; i < KPRE; ++i) pre[i] = lds_operand(kbuf, i, lane);   // K step 0 is in buffer 0
    for (; s < nT - 3; ++s) iteration(s, bool_tag<false>{}, bool_tag<true>{});
    for (; s < nT; ++s) iteration(s, bool_tag<true>{}, bool_tag<true>{});
  } else {
    for (; s < nT - 3; ++s) iteration(s, bool_tag<false>{}, bool_tag<false>{});
    for (; s < nT; ++s) iteration(s, bool_tag<true>{}, bool_tag<false>{});
  }
  if (group_b) {
    pv_tile<!VSMOOTH, true, !DUMP>(vbuf + ((nT - 1) & (NBUF - 1)) * TILE_BYTES, P, sb, one, O, L, lane, ones, bpre);
    if (VSMOOTH) {
      ofence(O);
      vsmooth_flush(mubuf, nT - 1, vinv, O, L, C, g, l16);
    }
  }
  {
    // O and L from the reference frame to the final running max (exact)
    ofence(O);
    float d0, d1;
    spread_pair(Mr - Mv, d0, d1);
    const int d[QBW] = {(int)d0, (int)d1};
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[qb][n][r] = __builtin_ldexpf(O[qb][n][r], d[qb]);
#pragma unroll
      for (int r = 0; r < 4; ++r) L[qb][r] = __builtin_ldexpf(L[qb][r], d[qb]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // Repair pass over the selected value tokens, with the final row max and
  // without touching L. Its sum R = sum_sel P r_hat has an accumulator of
  // its own (the scores' registers are free by now), so that the output
  // (sv*O + sr*R)/L needs no ratio of the two scales, which can leave the
  // fp32 range when the selected residuals are tiny against V.
  v4f R[QBW][8];
  const bool rep = REPAIR && a.n_sel > 0;
  if (REPAIR) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
      for (int n = 0; n < 8; ++n) R[qb][n] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  if (rep) {
    float M[QBW];   // final running max of each block, in every lane
    spread_pair(Mv, M[0], M[1]);
    const int nslot = a.n_sel_tiles * KTILE;
    const uint8_t* ksb = a.kselpack + (int64_t)bh * a.n_sel_tiles * TILE_BYTES;
    const uint8_t* rsb = a.rpack + (int64_t)bh * a.n_sel_tiles * TILE_BYTES;
    const float* sks = a.sksel + (int64_t)bh * nslot;
    for (int ts = 0; ts < a.n_sel_tiles; ++ts) {
      __syncthreads();   // every wave is done with the buffers about to be overwritten
      load_tile<NTHREADS>(kofs, ksb + (int64_t)ts * TILE_BYTES, voff, wvs);
      load_tile<NTHREADS>(vofs, rsb + (int64_t)ts * TILE_BYTES, voff, wvs);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const v8i kop = lds_operand(kbuf, kb, lane);
        float skk[4];
        bool live[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = ts * KTILE + 16 * kb + 4 * g + r;
          skk[r] = sks[slot];
          live[r] = slot < a.n_sel;
        }
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
          const v4f sc = mfma_f8(kop, qop[qb], v4f{0.f, 0.f, 0.f, 0.f});
          uint32_t w = 0;
          if (EXPP) {
            float e[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              e[r] = live[r] ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], aq[qb] * skk[r] * 0.125f, 8.0f - M[qb]))
                             : 0.0f;
            w = bytes_exp_fp8(e[0], e[1], e[2], e[3]);
          } else {
            const float bq = __builtin_fmaf(-8.0f, M[qb], EXPCAST_C);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float y = live[r] ? __builtin_fmaf(sc[r], aq[qb] * skk[r], bq) : -1.0f;
              w = __builtin_amdgcn_cvt_pk_u8_f32(y, r, w);
            }
          }
          P[qb][kb] = (int)w;
          if (DUMP && a.dump_rcodes != nullptr && dslot[qb] >= 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (live[r])
                a.dump_rcodes[(int64_t)dslot[qb] * a.n_sel + ts * KTILE + 16 * kb + 4 * g + r] = (uint8_t)(w >> (8 * r));
          }
        }
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const v8i rop = lds_operand(vbuf, n, lane);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) R[qb][n] = mfma_f8(rop, P[qb], R[qb][n]);
      }
    }
  }

  // ---- epilogue: out = (sv*O + sr*R) / L, BF16
  const float sv = a.sv[2 * bh];
  const float sr = rep ? a.sr[2 * bh] : 0.0f;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int qrow = q0 + 16 * qb + l16;
    if (qrow >= a.S) continue;
    const float fv = sv / L[qb][0], fr = sr / L[qb][0];
    uint16_t* orow = a.out + (((int64_t)b * a.S + qrow) * a.H + h) * HEAD_DIM + 4 * g;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = REPAIR ? __builtin_fmaf(R[qb][n][r], fr, O[qb][n][r] * fv) : O[qb][n][r] * fv;
      const uint32_t lo = f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16);
      const uint32_t hi = f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * n) = make_uint2(lo, hi);
      if (DUMP && a.dump_out32 != nullptr && dslot[qb] >= 0)
        *reinterpret_cast<float4*>(a.dump_out32 + (int64_t)dslot[qb] * HEAD_DIM + 16 * n + 4 * g) =
            make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}

template <bool REPAIR, bool DUMP, bool EXPP, bool VSMOOTH>
static hipError_t launch_one(const AttnArgs& a, dim3 grid, hipStream_t st) {
  constexpr int lds = VSMOOTH ? LDS_BYTES_VS : LDS_BYTES;
  static bool configured = false;
  if (!configured) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<REPAIR, DUMP, EXPP, VSMOOTH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL((attn_kernel<REPAIR, DUMP, EXPP, VSMOOTH>), grid, dim3(NTHREADS), lds, st, a);
  return hipGetLastError();
}

template <bool EXPP, bool VSMOOTH>
static hipError_t launch_variant(const AttnArgs& a, bool repair, bool dump, dim3 grid, hipStream_t st) {
  if (dump) return repair ? launch_one<true, true, EXPP, VSMOOTH>(a, grid, st) : launch_one<false, true, EXPP, VSMOOTH>(a, grid, st);
  return repair ? launch_one<true, false, EXPP, VSMOOTH>(a, grid, st) : launch_one<false, false, EXPP, VSMOOTH>(a, grid, st);
}

hipError_t launch_attention(const AttnArgs& args, bool repair, bool dump, hipStream_t st) {
  AttnArgs a = args;
  const int nwork = a.B * a.H * a.nQT;
  const int per = (nwork + 7) / 8;
  // Claiming pays for its atomics only when a CU runs many workgroups: at
  // 16 or more per CU (256 CUs), the last eighth of every XCD range is
  // claimed, by one and a half times as many workgroups, so that a faster
  // XCD can run up to 6% more than its own range.
  int per_xcd = per;
  a.sched_s0 = per;
  a.sched_n_claim = 0;
  if (!dump && nwork >= 16 * 256) {
    const int tail = per / 8, claimers = tail + tail / 2;
    a.sched_s0 = per - tail;
    a.sched_n_claim = 8 * claimers;
    per_xcd = a.sched_s0 + claimers;
  }
  const dim3 grid = dump ? dim3(a.nQT) : dim3(8 * per_xcd);
  if (a.vmu != nullptr)
    return a.exp_path ? launch_variant<true, true>(a, repair, dump, grid, st)
                      : launch_variant<false, true>(a, repair, dump, grid, st);
  return a.exp_path ? launch_variant<true, false>(a, repair, dump, grid, st)
                    : launch_variant<false, false>(a, repair, dump, grid, st);
}

}  // namespace oc
