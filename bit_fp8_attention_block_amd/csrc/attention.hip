// ExpCast FP8 attention kernel for gfx950.
//
// Method (VC-Attention write-up, "ExpCast-FP8" section; Open VC Attention
// product page, kernel paragraph): each softmax weight is written as its E4M3
// byte straight from the log-domain score with one FMA. No exponential is
// evaluated and no FP32->FP8 conversion is made. With a = 8*tau*log2(e)*sq*sk
// for the (query block, key tile) pair and the bit-aligned running row max M,
//     byte = clamp(rne(a*s_raw + (119.65 - 8*M)), 0, 255)
// is one v_fma_f32 and one v_cvt_pk_u8_f32 (which rounds to nearest even and
// clamps). The byte never exceeds 120 because M >= ceil(a*s_raw/8), and
// scores more than ~15 binades below the max land on 0.
//
// Because M is an integer, the weights of earlier tiles relative to a stale M
// differ from those relative to the new M by an exact power of two. The
// rescale is then an exact v_ldexp on O and L, and the result does not depend
// on the key-tile order (up to the underflow tail).
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
//    loads (global_load_lds_dwordx4), double-buffered. Their 16-byte
//    chunks are XOR-swizzled by row so operand reads are conflict-free.
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

// 32 operand bytes of `row`, k-slots 32g..32g+31, from a swizzled LDS tile
__device__ inline v8i lds_operand(const uint8_t* tile, int row, int g) {
  const uint4 x = *reinterpret_cast<const uint4*>(tile + swz(row, 32 * g));
  const uint4 y = *reinterpret_cast<const uint4*>(tile + swz(row, 32 * g + 16));
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

template <int NT>
__device__ inline void issue_tile_load(uint8_t* lds_buf, const uint8_t* ktile, const uint8_t* vtile) {
  // 32 KiB = 2048 chunks of 16 bytes; each instruction moves 1 KiB per wave,
  // lane l's chunk landing at wave base + 16*l
  const int tid = threadIdx.x, wv = tid >> 6;
#pragma unroll
  for (int i = 0; i < 2048 / NT; ++i) {
    const int ci = i * NT + tid;
    const uint8_t* src = (i * NT < 1024) ? ktile + ci * 16 : vtile + (ci - 1024) * 16;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_buf + (i * NT + wv * 64) * 16),
                                     16, 0, 0);
  }
}

__device__ inline float max_over_row_lanes(float m) {
  // the 4 lanes l, l^16, l^32, l^48 hold the same query
  const uint32_t u = __float_as_uint(m);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  m = __builtin_fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const uint32_t u2 = __float_as_uint(m);
  auto s32 = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
  return __builtin_fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

// QBW = 16-query blocks per wave; the workgroup has 16/QBW waves (256 queries)
template <int QBW, bool REPAIR, bool DUMP>
__global__ __launch_bounds__(1024 / QBW) void attn_kernel(AttnArgs a) {
  constexpr int NW = 16 / QBW;
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][2 * TILE_BYTES];

  int b, h, qt;
  if (DUMP) {
    b = a.dump_b; h = a.dump_h; qt = blockIdx.x;
  } else {
    // XCD-aware mapping: workgroup i runs on XCD i % 8; give each XCD a
    // contiguous range of (b, h, query tile) work items
    const int nwork = a.B * a.H * a.nQT;
    const int per = (nwork + 7) >> 3;
    const int w = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (w >= nwork) return;
    qt = w % a.nQT;
    const int bh_ = w / a.nQT;
    h = bh_ % a.H;
    b = bh_ / a.H;
  }
  const int bh = b * a.H + h;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int q0 = qt * BQ + wv * QBW * 16;
  const int nT = a.nT;

  // Q^T operands stay in registers for the whole loop
  v8i qop[QBW];
  float aq[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const uint8_t* p = a.qhat + ((int64_t)bh * a.s_pad_q + q0 + 16 * qb + l16) * HEAD_DIM + 32 * g;
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint4 y = *reinterpret_cast<const uint4*>(p + 16);
    qop[qb][0] = x.x; qop[qb][1] = x.y; qop[qb][2] = x.z; qop[qb][3] = x.w;
    qop[qb][4] = y.x; qop[qb][5] = y.y; qop[qb][6] = y.z; qop[qb][7] = y.w;
    aq[qb] = a.c8 * a.sq[(int64_t)bh * a.nQB + ((q0 + 16 * qb) >> 7)];
  }

  v4f O[8][QBW];
  v4f Lacc[QBW];
  float M[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    Lacc[qb] = v4f{0.f, 0.f, 0.f, 0.f};
    M[qb] = -16384.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) O[n][qb] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  v8i ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;   // E4M3 1.0

  const uint8_t* kbase = a.kpack + (int64_t)bh * nT * TILE_BYTES;
  const uint8_t* vbase = a.vpack + (int64_t)bh * nT * TILE_BYTES;
  const float* skp = a.sk + (int64_t)bh * nT;
  const int centre = (nT - 1) >> 1;
  const bool ragged = (a.S & (KTILE - 1)) != 0;

  {
    const int j0 = tile_at(0, centre, nT, a.order);
    issue_tile_load<NT>(smem[0], kbase + (int64_t)j0 * TILE_BYTES, vbase + (int64_t)j0 * TILE_BYTES);
  }
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0): this wave's tile chunks are in LDS
  __syncthreads();

  for (int s = 0; s < nT; ++s) {
    const int j = tile_at(s, centre, nT, a.order);
    const int buf = s & 1;
    if (s + 1 < nT) {
      const int jn = tile_at(s + 1, centre, nT, a.order);
      issue_tile_load<NT>(smem[buf ^ 1], kbase + (int64_t)jn * TILE_BYTES, vbase + (int64_t)jn * TILE_BYTES);
    }
    const uint8_t* kt = smem[buf];
    const uint8_t* vt = smem[buf] + TILE_BYTES;

    // ---- S^T = K Q^T for 128 keys x (16*QBW) queries
    v4f Sc[8][QBW];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const v8i kop = lds_operand(kt, 16 * kb + l16, g);
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) Sc[kb][qb] = mfma_f8(kop, qop[qb], v4f{0.f, 0.f, 0.f, 0.f});
    }
    if (ragged && j == nT - 1) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool dead = j * KTILE + 16 * kb + 4 * g + r >= a.S;
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb)
            if (dead) Sc[kb][qb][r] = -__builtin_inff();
        }
    }
    const float skj = skp[j];

    // ---- ExpCast: bytes straight from the scores
    v8i P[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      float m = Sc[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = __builtin_fmaxf(m, Sc[kb][qb][r]);
      m = max_over_row_lanes(m);
      const float al = aq[qb] * skj;
      const float mt = __builtin_ceilf((al * m) * 0.125f);
      const float Mn = __builtin_fmaxf(M[qb], mt);
      if (__builtin_amdgcn_ballot_w64(Mn > M[qb]) != 0) {
        const int d = (int)(M[qb] - Mn);   // <= 0
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[n][qb][r] = __builtin_ldexpf(O[n][qb][r], d);
#pragma unroll
        for (int r = 0; r < 4; ++r) Lacc[qb][r] = __builtin_ldexpf(Lacc[qb][r], d);
        M[qb] = Mn;
      }
      const float bq = __builtin_fmaf(-8.0f, Mn, EXPCAST_C);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(Sc[kb][qb][0], al, bq), 0, 0u);
        w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(Sc[kb][qb][1], al, bq), 1, w);
        w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(Sc[kb][qb][2], al, bq), 2, w);
        w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(Sc[kb][qb][3], al, bq), 3, w);
        P[qb][kb] = (int)w;
      }
      if (DUMP) {
        const int qrow = q0 + 16 * qb + l16;
        if (qrow < a.S) {
#pragma unroll
          for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = j * KTILE + 16 * kb + 4 * g + r;
              if (key < a.S) a.dump_codes[(int64_t)qrow * a.S + key] = (uint8_t)((uint32_t)P[qb][kb] >> (8 * r));
            }
          if (g == 0) a.dump_m[(int64_t)qrow * nT + j] = (int32_t)Mn;
        }
      }
    }

    // ---- O^T += V^T P^T ; L += 1 * P^T
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const v8i vop = lds_operand(vt, 16 * n + l16, g);
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) O[n][qb] = mfma_f8(vop, P[qb], O[n][qb]);
    }
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) Lacc[qb] = mfma_f8(ones, P[qb], Lacc[qb]);

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  float scale = a.sv[2 * bh];
  if (REPAIR && a.n_sel > 0) {
    // residual pass over the selected value tokens, with the final row max
    // and without touching L: O = sv*sum P v_hat + sr*sum P r_hat
    const float sr = a.sr[2 * bh];
    const float rs = scale / sr;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) O[n][qb] *= rs;
    scale = sr;
    const int nslot = a.n_sel_tiles * KTILE;
    const uint8_t* ksb = a.kselpack + (int64_t)bh * a.n_sel_tiles * TILE_BYTES;
    const uint8_t* rsb = a.rpack + (int64_t)bh * a.n_sel_tiles * TILE_BYTES;
    const float* sks = a.sksel + (int64_t)bh * nslot;
    for (int ts = 0; ts < a.n_sel_tiles; ++ts) {
      issue_tile_load<NT>(smem[0], ksb + (int64_t)ts * TILE_BYTES, rsb + (int64_t)ts * TILE_BYTES);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const uint8_t* kt = smem[0];
      const uint8_t* rt = smem[0] + TILE_BYTES;
      v8i P[QBW];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const v8i kop = lds_operand(kt, 16 * kb + l16, g);
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
          const float bq = __builtin_fmaf(-8.0f, M[qb], EXPCAST_C);
          uint32_t w = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float y = live[r] ? __builtin_fmaf(sc[r], aq[qb] * skk[r], bq) : -1.0f;
            w = __builtin_amdgcn_cvt_pk_u8_f32(y, r, w);
          }
          P[qb][kb] = (int)w;
        }
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const v8i rop = lds_operand(rt, 16 * n + l16, g);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) O[n][qb] = mfma_f8(rop, P[qb], O[n][qb]);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: out = O * scale / L, BF16
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int qrow = q0 + 16 * qb + l16;
    if (qrow >= a.S) continue;
    const float f = scale / Lacc[qb][0];
    uint16_t* orow = a.out + (((int64_t)b * a.S + qrow) * a.H + h) * HEAD_DIM + 4 * g;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint32_t lo = f32_to_bf16(O[n][qb][0] * f) | (f32_to_bf16(O[n][qb][1] * f) << 16);
      const uint32_t hi = f32_to_bf16(O[n][qb][2] * f) | (f32_to_bf16(O[n][qb][3] * f) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * n) = make_uint2(lo, hi);
    }
  }
}

template <int QBW>
static hipError_t launch_q(const AttnArgs& a, bool repair, bool dump, hipStream_t st) {
  const dim3 block(1024 / QBW);
  if (dump) {
    hipLaunchKernelGGL((attn_kernel<QBW, false, true>), dim3(a.nQT), block, 0, st, a);
  } else {
    const int nwork = a.B * a.H * a.nQT;
    const dim3 grid(8 * ((nwork + 7) / 8));
    if (repair) hipLaunchKernelGGL((attn_kernel<QBW, true, false>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<QBW, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool repair, bool dump, int qbw, hipStream_t st) {
  if (qbw == 2) return launch_q<2>(a, repair, dump, st);
  return launch_q<4>(a, repair, dump, st);
}

}  // namespace oc
