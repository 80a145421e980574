// Shared device-side definitions of the ExpCast FP8 attention library:
// tile geometry, workspace pack layouts and the E4M3 helpers used by the
// prepare and attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oc {

constexpr int HEAD_DIM = 128;
constexpr int KTILE = 128;        // keys per tile = Q/K scale block
constexpr int BQ = 256;           // queries per attention workgroup
constexpr int TILE_BYTES = KTILE * HEAD_DIM;   // one FP8 tile: 16 KiB
constexpr int SCHED_WORDS = 16;  // attention work-item counters: 8 XCD ranges, a claim count, padding

// ExpCast constant: byte = rne(8*(x - M) + 120 + beta), beta = -0.35
// (VC-Attention write-up, "ExpCast-FP8" section; 120 is the E4M3 byte of 256).
constexpr float EXPCAST_C = 119.65f;
constexpr float E4M3_MAX = 448.0f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// ---- pack layouts (workspace format, documented in oc_attn.h) ----

// Byte offset of (row, column) inside a 128x128 FP8 tile stored in MFMA
// operand order. The 16x16x128 FP8 MFMA takes, in lane l, 32 bytes of row
// l%16 of a 16-row block: columns 32*(l/16) .. +32, as two 16-byte halves.
// The tile is stored so that the half h of 16-row block kb for lane l is the
// 16-byte chunk (2*kb + h)*64 + l: an operand read is then one contiguous
// 1 KiB ds_read_b128 per wave (the only bank-conflict-free b128 pattern on
// gfx950), and the global->LDS copy of a tile stays a straight copy.
__host__ __device__ inline int opidx(int row, int col) {
  const int c = col >> 4;                              // 16-byte chunk of the row
  const int lane = ((c >> 1) << 4) | (row & 15);
  return ((((row >> 4) << 1) | (c & 1)) * 64 + lane) * 16 + (col & 15);
}

// Column of key j (0..127) in a transposed V tile. The QK^T MFMA output leaves
// lane l holding keys 16t + 4g + r (g = l/16, t = 0..7, r = 0..3) of one query;
// those 32 bytes become the B operand of the PV MFMA, whose lane l consumes
// k-slots 32g..32g+31. So key 16t+4g+r must sit at slot 32g + 4t + r.
__host__ __device__ inline int vcol_of_key(int j) {
  return 32 * ((j >> 2) & 3) + 4 * (j >> 4) + (j & 3);
}

// ---- E4M3 (OCP, no infinities) ----

// Exact decode of a byte code to fp32.
__device__ inline float e4m3_decode(uint32_t c) {
  uint32_t mag = c & 0x7Fu;
  float v = (mag < 8u) ? (float)mag * 0.001953125f
                       : __uint_as_float((((mag >> 3) + 120u) << 23) | ((mag & 7u) << 20));
  return (c & 0x80u) ? -v : v;
}

// Two fp32 values -> two E4M3 bytes (low 16 bits of the result), nearest
// value with ties to the even code, saturating at +-448. The hardware
// conversion rounds to nearest even but does not saturate, so clamp first.
__device__ inline uint32_t e4m3_encode2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -E4M3_MAX), E4M3_MAX);
  b = __builtin_fminf(__builtin_fmaxf(b, -E4M3_MAX), E4M3_MAX);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// 16-bit float payloads -> fp32
__device__ inline float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ inline float f16_to_f32(uint32_t h) {
  _Float16 x;
  uint16_t hb = (uint16_t)h;
  __builtin_memcpy(&x, &hb, 2);
  return (float)x;
}
template <bool FP16>
__device__ inline float half_to_f32(uint32_t h) {
  return FP16 ? f16_to_f32(h) : bf16_to_f32(h);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Quantization scales from a block amax: s = amax/448, inv = 448/amax
// (correctly rounded fp32 divisions). A block whose amax is below 2^-100, an
// all-zero block included, gets (1, 1): every element then rounds to code 0,
// and 448/amax, which leaves the fp32 range below about 1.3e-36, is never
// formed. From 2^-100 up both quotients are normal numbers.
constexpr float SCALE_FLOOR = 0x1p-100f;
__device__ inline void quant_scales(float amax, float& s, float& inv) {
  if (amax < SCALE_FLOOR) { s = 1.0f; inv = 1.0f; return; }
  s = __fdiv_rn(amax, E4M3_MAX);
  inv = __fdiv_rn(E4M3_MAX, amax);
}

// ---- wave / block reductions ----
__device__ inline float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace oc
