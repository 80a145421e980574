// Prepare kernels: BF16/FP16 Q, K, V -> E4M3 codes and scales in the
// workspace, plus the V-residual repair set.
//
// Follows the Open VC Attention product page (kernel paragraph: per-block Q/K
// scales, per-head V scale, V packed transposed for the matrix cores) and the
// Open-VC news page ("Архитектурные оптимизации": input preparation fused
// into one graph; "Решение: ExpCast ...": residual repair of the worst-rounded
// value tokens). All four kernels are memory-bound; see oc_attn.h for the
// workspace layouts they write.
#include "oc_common.h"
#include "oc_kernels.h"

namespace oc {

// Load 16 consecutive 16-bit channels [16*oc, 16*oc+16) of one token, or
// zeros for a token beyond S.
__device__ inline void load16(const uint16_t* base, bool valid, uint4& lo, uint4& hi) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if (valid) {
    const u32x4* p = reinterpret_cast<const u32x4*>(base);
    const u32x4 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 1);
    lo = make_uint4(x[0], x[1], x[2], x[3]);
    hi = make_uint4(y[0], y[1], y[2], y[3]);
  } else {
    lo = make_uint4(0, 0, 0, 0);
    hi = lo;
  }
}

// max |x| bit pattern over 16 packed halves (sign dropped; bf16 and fp16
// magnitudes order like their bit patterns)
__device__ inline uint32_t absmax_bits(uint4 lo, uint4 hi, uint32_t m) {
  uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t x = w[i] & 0x7FFF7FFFu;
    m = max(m, max(x & 0xFFFFu, x >> 16));
  }
  return m;
}

template <bool FP16>
__device__ inline float bits_to_f32(uint32_t h) { return half_to_f32<FP16>(h); }

// 16 halves -> 16 E4M3 bytes of x * inv
template <bool FP16>
__device__ inline uint4 encode16(uint4 lo, uint4 hi, float inv) {
  uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = w[2 * i], b = w[2 * i + 1];
    uint32_t p0 = e4m3_encode2(bits_to_f32<FP16>(a & 0xFFFFu) * inv, bits_to_f32<FP16>(a >> 16) * inv);
    uint32_t p1 = e4m3_encode2(bits_to_f32<FP16>(b & 0xFFFFu) * inv, bits_to_f32<FP16>(b >> 16) * inv);
    o[i] = p0 | (p1 << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// block-wide max of a non-negative value (blockDim.x threads, <= 1024)
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = 0.0f;
  for (int i = 0; i < nw; ++i) m = __builtin_fmaxf(m, red[i]);
  return m;
}

// 16 fp32 values -> 16 E4M3 bytes of x * inv
__device__ inline uint4 encode16f(const float (&x)[16], float inv) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p0 = e4m3_encode2(x[4 * i] * inv, x[4 * i + 1] * inv);
    const uint32_t p1 = e4m3_encode2(x[4 * i + 2] * inv, x[4 * i + 3] * inv);
    o[i] = p0 | (p1 << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// K-mean smoothing, step 1: per (b, h, 128-token block), the float64 sum of
// the block's keys per channel (exact for bf16/fp16 inputs unless a channel
// spans more than about 28 binades). grid (nT, H, B), 256 threads.
template <bool FP16>
__global__ __launch_bounds__(256) void kmean_partial_kernel(PrepArgs a) {
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, rsub = tid >> 3, oc = tid & 7;
  const int bh = b * a.H + h;
  __shared__ double part[32][HEAD_DIM + 1];
  double acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int tok = blk * KTILE + 32 * p + rsub;
    const int64_t off = (int64_t)b * a.sb + (int64_t)tok * a.ss + (int64_t)h * a.sh + 16 * oc;
    uint4 lo, hi;
    load16(a.k + off, tok < a.S, lo, hi);
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[2 * i] += (double)half_to_f32<FP16>(w[i] & 0xFFFFu);
      acc[2 * i + 1] += (double)half_to_f32<FP16>(w[i] >> 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) part[rsub][16 * oc + i] = acc[i];
  __syncthreads();
  if (tid < HEAD_DIM) {
    double t = 0.0;
    for (int r = 0; r < 32; ++r) t += part[r][tid];
    a.kpart[((int64_t)bh * a.nT + blk) * HEAD_DIM + tid] = t;
  }
}

// K-mean smoothing, step 2: per (b, h), kbar = fp32(sum / S) per channel.
// grid (H, B), 1024 threads: 8 groups of 128 channels take every 8th block,
// then the 8 group sums are added in group order.
__global__ __launch_bounds__(1024) void kmean_final_kernel(PrepArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, bh = b * a.H + h;
  const int g = threadIdx.x >> 7, c = threadIdx.x & (HEAD_DIM - 1);
  __shared__ double part[8][HEAD_DIM];
  double t = 0.0;
  for (int blk = g; blk < a.nT; blk += 8) t += a.kpart[((int64_t)bh * a.nT + blk) * HEAD_DIM + c];
  part[g][c] = t;
  __syncthreads();
  if (g == 0) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += part[i][c];
    a.kmean[(int64_t)bh * HEAD_DIM + c] = (float)(s / (double)a.S);
  }
}

// ---------------------------------------------------------------------------
// Kernel 1: per (b, h, 128-token block): Q and K block amax, scales, codes;
// V block amax (the per-head V scale needs all blocks first). With
// KSMOOTH the keys are fp32(k - kbar) before their block amax and codes.
// With VSMOOTH the block's V mean mu = bf16(fp32(sum / n)) per channel (sum in
// float64 over the n valid tokens) is stored, and the V amax is that of the
// residuals fp32(v - mu).
// grid (nQB, H, B), 256 threads; thread -> rows {32p + tid/8}, channels 16*(tid%8)..+16
template <bool FP16, bool KSMOOTH, bool VSMOOTH>
__global__ __launch_bounds__(256) void prep_qk_kernel(PrepArgs a) {
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, rsub = tid >> 3, oc = tid & 7;
  const int bh = b * a.H + h;
  const bool kv = blk < a.nT;
  __shared__ float red[16];
  // the attention kernel's work-item counters start at zero
  if ((blk | h | b) == 0 && tid < SCHED_WORDS) a.sched[tid] = 0u;

  uint4 ql[4], qh[4], kl[4], kh[4], vl[4], vh[4];
  uint32_t mq = 0, mk = 0, mv = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int tok = blk * KTILE + 32 * p + rsub;
    const bool valid = tok < a.S;
    const int64_t off = (int64_t)b * a.sb + (int64_t)tok * a.ss + (int64_t)h * a.sh + 16 * oc;
    load16(a.q + off, valid, ql[p], qh[p]);
    mq = absmax_bits(ql[p], qh[p], mq);
    load16(a.k + off, valid && kv, kl[p], kh[p]);
    mk = absmax_bits(kl[p], kh[p], mk);
    load16(a.v + off, valid && kv, vl[p], vh[p]);
    mv = absmax_bits(vl[p], vh[p], mv);
  }
  float amv_local = bits_to_f32<FP16>(mv);
  if (VSMOOTH && kv) {
    // block mean per channel: per-thread sums of its 4 rows (padding rows are
    // zero), then the 32 row groups in order
    __shared__ double vsum[32][HEAD_DIM + 1];
    __shared__ float vmu_s[HEAD_DIM];
    double acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w[8] = {vl[p].x, vl[p].y, vl[p].z, vl[p].w, vh[p].x, vh[p].y, vh[p].z, vh[p].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[2 * i] += (double)bits_to_f32<FP16>(w[i] & 0xFFFFu);
        acc[2 * i + 1] += (double)bits_to_f32<FP16>(w[i] >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) vsum[rsub][16 * oc + i] = acc[i];
    __syncthreads();
    if (tid < HEAD_DIM) {
      double t = 0.0;
      for (int r = 0; r < 32; ++r) t += vsum[r][tid];
      const int n = min(KTILE, a.S - blk * KTILE);
      const uint32_t hb = f32_to_bf16((float)(t / (double)n));
      vmu_s[tid] = bf16_to_f32(hb);
      a.vmu[((int64_t)bh * a.nT + blk) * HEAD_DIM + tid] = (uint16_t)hb;
    }
    __syncthreads();
    amv_local = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool valid = blk * KTILE + 32 * p + rsub < a.S;
      const uint32_t w[8] = {vl[p].x, vl[p].y, vl[p].z, vl[p].w, vh[p].x, vh[p].y, vh[p].z, vh[p].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r0 = bits_to_f32<FP16>(w[i] & 0xFFFFu) - vmu_s[16 * oc + 2 * i];
        const float r1 = bits_to_f32<FP16>(w[i] >> 16) - vmu_s[16 * oc + 2 * i + 1];
        if (valid) amv_local = __builtin_fmaxf(amv_local, __builtin_fmaxf(__builtin_fabsf(r0), __builtin_fabsf(r1)));
      }
    }
  }
  float ks[KSMOOTH ? 4 : 1][16];
  float amk_local = bits_to_f32<FP16>(mk);
  if (KSMOOTH) {
    float kbar[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kbar[i] = a.kmean[(int64_t)bh * HEAD_DIM + 16 * oc + i];
    amk_local = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bool valid = blk * KTILE + 32 * p + rsub < a.S;
      const uint32_t w[8] = {kl[p].x, kl[p].y, kl[p].z, kl[p].w, kh[p].x, kh[p].y, kh[p].z, kh[p].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // padding rows stay zero
        ks[p][2 * i] = valid ? bits_to_f32<FP16>(w[i] & 0xFFFFu) - kbar[2 * i] : 0.0f;
        ks[p][2 * i + 1] = valid ? bits_to_f32<FP16>(w[i] >> 16) - kbar[2 * i + 1] : 0.0f;
        amk_local = __builtin_fmaxf(amk_local, __builtin_fmaxf(__builtin_fabsf(ks[p][2 * i]),
                                                               __builtin_fabsf(ks[p][2 * i + 1])));
      }
    }
  }
  const float amq = block_max(bits_to_f32<FP16>(mq), red);
  const float amk = block_max(amk_local, red + 4);
  const float amv = block_max(amv_local, red + 8);
  float sq, iq, sk, ik;
  quant_scales(amq, sq, iq);
  quant_scales(amk, sk, ik);
  if (tid == 0) {
    a.sq[(int64_t)bh * a.nQB + blk] = sq;
    if (kv) {
      a.sk[(int64_t)bh * a.nT + blk] = sk;
      a.vamax[(int64_t)bh * a.nT + blk] = amv;
    }
  }
  uint8_t* qdst = a.qhat + ((int64_t)bh * a.s_pad_q + (int64_t)blk * KTILE) * HEAD_DIM;
  uint8_t* kdst = a.kpack + ((int64_t)bh * a.nT + blk) * TILE_BYTES;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = 32 * p + rsub;
    *reinterpret_cast<uint4*>(qdst + row * HEAD_DIM + 16 * oc) = encode16<FP16>(ql[p], qh[p], iq);
    if (kv) {
      uint4 kc;
      if (KSMOOTH) kc = encode16f(ks[p], ik);
      else kc = encode16<FP16>(kl[p], kh[p], ik);
      *reinterpret_cast<uint4*>(kdst + opidx(row, 16 * oc)) = kc;
    }
  }
}

// ---------------------------------------------------------------------------
// 16 halves minus 16 per-channel fp32 offsets -> 16 E4M3 bytes of fp32(x - mu) * inv
template <bool FP16>
__device__ inline uint4 encode16_sub(uint4 lo, uint4 hi, const float (&mu)[16], float inv) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bits_to_f32<FP16>(w[i] & 0xFFFFu) - mu[2 * i];
    x[2 * i + 1] = bits_to_f32<FP16>(w[i] >> 16) - mu[2 * i + 1];
  }
  return encode16f(x, inv);
}

// Kernel 2: per (b, h, key tile): head V scale from the block maxima, V codes
// transposed and packed into the PV operand order (through LDS), and with
// repair the residual energy of every token. With VSMOOTH the codes are of
// fp32(v - mu) for the tile's block mean mu, and mu * inv is stored in the
// order the attention kernel's mean-term MFMA reads it.
// grid (nT, H, B), 256 threads; thread -> tokens 4m..4m+3 (m = tid/8), channels 16*(tid%8)..+16
template <bool FP16, bool REPAIR, bool VSMOOTH>
__global__ __launch_bounds__(256) void prep_v_kernel(PrepArgs a) {
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, m = tid >> 3, oc = tid & 7;
  const int bh = b * a.H + h;
  __shared__ float red[16];
  __shared__ __attribute__((aligned(16))) uint8_t lds[TILE_BYTES];

  float mx = 0.0f;
  for (int i = tid; i < a.nT; i += 256) mx = __builtin_fmaxf(mx, a.vamax[(int64_t)bh * a.nT + i]);
  const float amax = block_max(mx, red);
  float sv, inv;
  quant_scales(amax, sv, inv);
  if (tile == 0 && tid == 0) {
    a.sv[2 * bh] = sv;
    a.sv[2 * bh + 1] = inv;
  }

  float mu[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
    mu[c] = VSMOOTH ? bf16_to_f32(a.vmu[((int64_t)bh * a.nT + tile) * HEAD_DIM + 16 * oc + c]) : 0.0f;
  uint4 lo[4], hi[4], cd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = tile * KTILE + 4 * m + r;
    const int64_t off = (int64_t)b * a.sb + (int64_t)tok * a.ss + (int64_t)h * a.sh + 16 * oc;
    load16(a.v + off, tok < a.S, lo[r], hi[r]);
    if (VSMOOTH) cd[r] = tok < a.S ? encode16_sub<FP16>(lo[r], hi[r], mu, inv) : make_uint4(0, 0, 0, 0);
    else cd[r] = encode16<FP16>(lo[r], hi[r], inv);
  }
  // transpose: channel d = 16*oc + c gets the 4 bytes of tokens 4m..4m+3,
  // which sit in 4 consecutive columns of the packed tile
  const int kcol = vcol_of_key(4 * m);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint32_t sh = 8 * (c & 3);
    const int wsel = c >> 2;
    uint32_t w = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t word = (wsel == 0) ? cd[r].x : (wsel == 1) ? cd[r].y : (wsel == 2) ? cd[r].z : cd[r].w;
      w |= ((word >> sh) & 0xFFu) << (8 * r);
    }
    *reinterpret_cast<uint32_t*>(lds + opidx(16 * oc + c, kcol)) = w;
  }
  __syncthreads();
  uint8_t* dst = a.vpack + ((int64_t)bh * a.nT + tile) * TILE_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = (i * 256 + tid) * 16;
    *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(lds + o);
  }

  if (REPAIR) {
    // residual r = v - sv*dec(code) in fp32 (two roundings, no fusion);
    // energy = sum of r^2 over the 128 channels in float64, added pairwise in
    // channel order: each square is exact, a four-level tree adds this
    // thread's 16 channels (an aligned block of the channel order), and the
    // xor exchanges over the 8 threads of the token are the tree's top three
    // levels (a + b == b + a, so every thread ends with the same bits)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t w[8] = {lo[r].x, lo[r].y, lo[r].z, lo[r].w, hi[r].x, hi[r].y, hi[r].z, hi[r].w};
      const uint32_t cw[4] = {cd[r].x, cd[r].y, cd[r].z, cd[r].w};
      // decoded codes (the hardware E4M3 -> fp32 conversion is exact)
      float dec[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v2f lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[j], false);
        const v2f hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[j], true);
        dec[4 * j] = lo2[0]; dec[4 * j + 1] = lo2[1]; dec[4 * j + 2] = hi2[0]; dec[4 * j + 3] = hi2[1];
      }
      double e2[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float x = __fsub_rn(bits_to_f32<FP16>((w[c >> 1] >> (16 * (c & 1))) & 0xFFFFu), mu[c]);
        const float t = __fmul_rn(sv, dec[c]);
        const double d = (double)__fsub_rn(x, t);
        e2[c] = d * d;
      }
#pragma unroll
      for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
        for (int i = 0; i < n; ++i) e2[i] = e2[2 * i] + e2[2 * i + 1];
      double e = e2[0];
      e += __shfl_xor(e, 1, 64);
      e += __shfl_xor(e, 2, 64);
      e += __shfl_xor(e, 4, 64);
      const int tok = tile * KTILE + 4 * m + r;
      if (oc == 0 && tok < a.S) a.energy[(int64_t)bh * a.S + tok] = e;
    }
  }
}

// ---------------------------------------------------------------------------
// block-wide exclusive prefix sum (1024 threads)
__device__ inline int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) scratch[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += scratch[i];
    tot += scratch[i];
  }
  total = tot;
  return before + x - v;
}

// V-Smooth block mean of channel c for token tok (0 without smoothing)
__device__ inline float vmean_of(const PrepArgs& a, int bh, int tok, int c) {
  return a.vmu ? bf16_to_f32(a.vmu[((int64_t)bh * a.nT + (tok >> 7)) * HEAD_DIM + c]) : 0.0f;
}

// residual of one value element, recomputed exactly as prep_v_kernel does
// (mu: the element's V-Smooth block mean, 0 without smoothing)
template <bool FP16>
__device__ inline float residual(uint32_t hbits, float mu, float sv, float inv) {
  const float x = __fsub_rn(bits_to_f32<FP16>(hbits), mu);
  const uint32_t code = e4m3_encode2(x * inv, 0.0f) & 0xFFu;
  return __fsub_rn(x, __fmul_rn(sv, e4m3_decode(code)));
}

// ---------------------------------------------------------------------------
// Kernel 3: per (b, h): top-k tokens by residual energy (radix select on the
// float64 bit patterns, which order like the non-negative values), ties to
// the lower index, written in ascending token order; then the amax of the
// selected residuals gives the residual scale.
// grid (H, B), 1024 threads
template <bool FP16>
__global__ __launch_bounds__(1024) void select_kernel(PrepArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int bh = b * a.H + h;
  const int S = a.S, k = a.n_sel;
  const uint64_t* e = reinterpret_cast<const uint64_t*>(a.energy + (int64_t)bh * S);
  __shared__ uint32_t hist[256];
  __shared__ uint32_t above[256];   // tokens in higher bins, by bin
  __shared__ int scratch[16];
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem, s_all;
  __shared__ float red[16];

  uint64_t prefix = 0, mask = 0;
  int krem = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    // a thread counts runs of equal digits before adding them: the leading
    // digits of the energies are nearly all alike, and one LDS atomic per
    // token on a handful of bins would serialise the whole block. Loads go
    // out eight at a time (one latency per batch, not per token).
    uint32_t run_bin = 256u, run = 0u;
    for (int i0 = 0; i0 < S; i0 += 8 * 1024) {
      uint64_t u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + j * 1024 + tid;
        u[j] = i < S ? e[i] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (i0 + j * 1024 + tid >= S || (u[j] & mask) != prefix) continue;
        const uint32_t bin = (uint32_t)(u[j] >> shift) & 255u;
        if (bin != run_bin) {
          if (run) atomicAdd(&hist[run_bin], run);
          run_bin = bin;
          run = 0u;
        }
        ++run;
      }
    }
    if (run) atomicAdd(&hist[run_bin], run);
    __syncthreads();
    // the bin of the krem-th largest: above[b] = tokens in bins > b (an
    // inclusive suffix scan over the 256 bins, 8 steps), then the one bin with
    // above[b] < krem <= above[b] + hist[b]
    if (tid < 256) above[tid] = hist[tid];
    __syncthreads();
#pragma unroll
    for (int d = 1; d < 256; d <<= 1) {
      const uint32_t add = tid < 256 && tid + d < 256 ? above[tid + d] : 0u;
      __syncthreads();
      if (tid < 256) above[tid] += add;
      __syncthreads();
    }
    if (tid < 256) {
      const int gt = (int)(above[tid] - hist[tid]);
      if (gt < krem && krem <= (int)above[tid]) {
        s_prefix = prefix | ((uint64_t)tid << shift);
        s_krem = krem - gt;
        s_all = (int)hist[tid] == krem - gt;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= (uint64_t)255 << shift;
    // every token whose leading bits equal the prefix is taken: the set is
    // settled, and finer digits would not change it
    if (s_all) break;
    __syncthreads();
  }
  // prefix = the leading bits (under mask) of the k-th largest energy T;
  // krem = how many tokens with those bits to take (all of them when the
  // passes stopped early)
  const int chunk = (S + 1023) / 1024;
  const int i0 = min(S, tid * chunk), i1 = min(S, i0 + chunk);
  int gt = 0, eq = 0;
  for (int ib = i0; ib < i1; ib += 8) {
    uint64_t u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = ib + j < i1 ? e[ib + j] : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      gt += ib + j < i1 && (u[j] & mask) > prefix;
      eq += ib + j < i1 && (u[j] & mask) == prefix;
    }
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, scratch, tot);
  const int take_eq = max(0, min(eq, krem - eq_before));
  int pos = block_exclusive_scan(gt + take_eq, scratch, tot);
  int32_t* sel = a.sel + (int64_t)bh * a.n_sel;
  int taken = 0;
  if (gt + take_eq > 0) {
    for (int ib = i0; ib < i1; ib += 8) {
      uint64_t u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = ib + j < i1 ? e[ib + j] : 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t um = u[j] & mask;
        if (ib + j < i1 && (um > prefix || (um == prefix && taken < take_eq))) {
          sel[pos++] = ib + j;
          if (um == prefix) ++taken;
        }
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // residual amax over the selected tokens (8-channel chunks)
  const float sv = a.sv[2 * bh], inv = a.sv[2 * bh + 1];
  float mx = 0.0f;
  for (int64_t it = tid; it < (int64_t)k * 16; it += 1024) {
    const int slot = (int)(it >> 4), c8 = (int)(it & 15) * 8;
    const int tok = sel[slot];
    const int64_t off = (int64_t)b * a.sb + (int64_t)tok * a.ss + (int64_t)h * a.sh + c8;
    const uint4 w = *reinterpret_cast<const uint4*>(a.v + off);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float r = residual<FP16>((ws[c >> 1] >> (16 * (c & 1))) & 0xFFFFu, vmean_of(a, bh, tok, c8 + c), sv, inv);
      mx = __builtin_fmaxf(mx, __builtin_fabsf(r));
    }
  }
  const float amax = block_max(mx, red);
  if (tid == 0) {
    float s, i;
    quant_scales(amax, s, i);
    a.sr[2 * bh] = s;
    a.sr[2 * bh + 1] = i;
  }
}

// ---------------------------------------------------------------------------
// Kernel 4: per (b, h, slot tile): gather the selected K rows (codes and
// block scales) and pack the E4M3 residuals like V.
// grid (nTs, H, B), 256 threads
template <bool FP16>
__global__ __launch_bounds__(256) void pack_repair_kernel(PrepArgs a) {
  const int ts = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int bh = b * a.H + h;
  const int k = a.n_sel;
  const int nslot = a.n_sel_tiles * KTILE;
  const int32_t* sel = a.sel + (int64_t)bh * a.n_sel;
  __shared__ __attribute__((aligned(16))) uint8_t lds[TILE_BYTES];

  // K rows: thread -> slot tid/2, chunks 4*(tid%2)..+4
  {
    const int sl = tid >> 1, half = tid & 1;
    const int slot = ts * KTILE + sl;
    uint8_t* dst = a.kselpack + ((int64_t)bh * a.n_sel_tiles + ts) * TILE_BYTES;
    if (slot < k) {
      const int j = sel[slot];
      const uint8_t* src = a.kpack + ((int64_t)bh * a.nT + (j >> 7)) * TILE_BYTES;
      const int sr = j & 127;
#pragma unroll
      for (int c = 4 * half; c < 4 * half + 4; ++c)
        *reinterpret_cast<uint4*>(dst + opidx(sl, 16 * c)) = *reinterpret_cast<const uint4*>(src + opidx(sr, 16 * c));
      if (half == 0) a.sksel[(int64_t)bh * nslot + slot] = a.sk[(int64_t)bh * a.nT + (j >> 7)];
    } else {
#pragma unroll
      for (int c = 4 * half; c < 4 * half + 4; ++c)
        *reinterpret_cast<uint4*>(dst + opidx(sl, 16 * c)) = make_uint4(0, 0, 0, 0);
      if (half == 0) a.sksel[(int64_t)bh * nslot + slot] = 0.0f;
    }
  }
  // residual codes, transposed like V: thread -> slots 4m..4m+3, channels 16*oc..+16
  const int m = tid >> 3, oc = tid & 7;
  const float sv = a.sv[2 * bh], inv = a.sv[2 * bh + 1];
  const float rinv = a.sr[2 * bh + 1];
  uint32_t cw[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = ts * KTILE + 4 * m + r;
    uint4 lo, hi;
    const int tok = slot < k ? sel[slot] : 0;
    const int64_t off = (int64_t)b * a.sb + (int64_t)tok * a.ss + (int64_t)h * a.sh + 16 * oc;
    load16(a.v + off, slot < k, lo, hi);
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = 16 * oc + 4 * q;
      const float r0 = residual<FP16>(w[2 * q] & 0xFFFFu, vmean_of(a, bh, tok, c0), sv, inv) * rinv;
      const float r1 = residual<FP16>(w[2 * q] >> 16, vmean_of(a, bh, tok, c0 + 1), sv, inv) * rinv;
      const float r2 = residual<FP16>(w[2 * q + 1] & 0xFFFFu, vmean_of(a, bh, tok, c0 + 2), sv, inv) * rinv;
      const float r3 = residual<FP16>(w[2 * q + 1] >> 16, vmean_of(a, bh, tok, c0 + 3), sv, inv) * rinv;
      cw[r][q] = e4m3_encode2(r0, r1) | (e4m3_encode2(r2, r3) << 16);
    }
  }
  const int kcol = vcol_of_key(4 * m);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    uint32_t w = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) w |= ((cw[r][c >> 2] >> (8 * (c & 3))) & 0xFFu) << (8 * r);
    *reinterpret_cast<uint32_t*>(lds + opidx(16 * oc + c, kcol)) = w;
  }
  __syncthreads();
  uint8_t* dst = a.rpack + ((int64_t)bh * a.n_sel_tiles + ts) * TILE_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = (i * 256 + tid) * 16;
    *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(lds + o);
  }
}

// ---------------------------------------------------------------------------
template <bool FP16, bool VSMOOTH>
static void launch_qk(const PrepArgs& a, hipStream_t st) {
  const dim3 g1(a.nQB, a.H, a.B), g2(a.nT, a.H, a.B);
  if (a.kmean != nullptr) {
    hipLaunchKernelGGL(kmean_partial_kernel<FP16>, g2, dim3(256), 0, st, a);
    hipLaunchKernelGGL(kmean_final_kernel, dim3(a.H, a.B), dim3(1024), 0, st, a);
    hipLaunchKernelGGL((prep_qk_kernel<FP16, true, VSMOOTH>), g1, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((prep_qk_kernel<FP16, false, VSMOOTH>), g1, dim3(256), 0, st, a);
  }
}

template <bool FP16, bool VSMOOTH>
static void launch_qkv(const PrepArgs& a, hipStream_t st) {
  const dim3 g2(a.nT, a.H, a.B);
  launch_qk<FP16, VSMOOTH>(a, st);
  if (a.energy != nullptr) hipLaunchKernelGGL((prep_v_kernel<FP16, true, VSMOOTH>), g2, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((prep_v_kernel<FP16, false, VSMOOTH>), g2, dim3(256), 0, st, a);
}

hipError_t launch_prepare(const PrepArgs& a, bool fp16, hipStream_t st) {
  const bool rep = a.energy != nullptr, vs = a.vmu != nullptr;
  if (fp16) {
    if (vs) launch_qkv<true, true>(a, st);
    else launch_qkv<true, false>(a, st);
  } else {
    if (vs) launch_qkv<false, true>(a, st);
    else launch_qkv<false, false>(a, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !rep || a.n_sel == 0) return e;
  const dim3 g3(a.H, a.B), g4(a.n_sel_tiles, a.H, a.B);
  if (fp16) {
    hipLaunchKernelGGL(select_kernel<true>, g3, dim3(1024), 0, st, a);
    hipLaunchKernelGGL(pack_repair_kernel<true>, g4, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(select_kernel<false>, g3, dim3(1024), 0, st, a);
    hipLaunchKernelGGL(pack_repair_kernel<false>, g4, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace oc
