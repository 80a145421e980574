// Kernel argument blocks and launchers shared by the host library and the
// kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oc {

struct PrepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, ss, sh;          // element strides shared by q, k, v
  int B, S, H;
  int nT, nQB, s_pad_q;        // key tiles, Q scale blocks, padded Q rows
  uint8_t* qhat;
  uint8_t* kpack;
  uint8_t* vpack;
  float* sq;
  float* sk;
  float* vamax;
  float* sv;                   // [B][H][2]: amax/448, 448/amax
  // K-mean smoothing (kmean == nullptr: off)
  float* kmean;                // [B][H][128] fp32 mean key
  double* kpart;               // [B][H][nT][128] per-block key sums
  // V-Smooth block means (vmu == nullptr: off)
  uint16_t* vmu;               // [B][H][nT][128] bf16 block means
  // repair (energy == nullptr: no repair)
  double* energy;
  int32_t* sel;
  uint8_t* kselpack;
  uint8_t* rpack;
  float* sksel;
  float* sr;                   // [B][H][2]
  int n_sel, n_sel_tiles;
  uint32_t* sched;             // [SCHED_WORDS] attention work-item counters, zeroed here
};

struct AttnArgs {
  const uint8_t* qhat;
  const uint8_t* kpack;
  const uint8_t* vpack;
  const float* sq;
  const float* sk;
  const float* sv;
  const uint8_t* kselpack;
  const uint8_t* rpack;
  const float* sksel;
  const float* sr;
  int n_sel, n_sel_tiles;
  uint16_t* out;               // bf16 [B][S][H][128], contiguous
  int B, S, H, nT, nQT, nQB, s_pad_q;
  float c8;                    // 8 * tau * log2(e)
  int order;                   // 0: from the middle of the key window outwards, 1: ascending
  int exp_path;                // 0: ExpCast bytes; 1: exp2 + FP32->E4M3 cast (comparison path)
  const uint16_t* vmu;         // V-Smooth: [B][H][nT][128] bf16 block means (nullptr: off)
  // parity aid (the DUMP variant only): one (b, h), the listed query rows
  const int32_t* dump_rows;    // [n_dump] ascending query rows
  int n_dump;
  uint8_t* dump_codes;         // [n_dump][S] main-loop bytes (or nullptr)
  int32_t* dump_m;             // [n_dump][nT] running max per key tile (or nullptr)
  float* dump_scores;          // [n_dump][S] raw MFMA sums <q_hat, k_hat> (or nullptr)
  uint8_t* dump_rcodes;        // [n_dump][n_sel] repair-pass bytes (or nullptr)
  float* dump_out32;           // [n_dump][128] fp32 output before BF16 rounding (or nullptr)
  int dump_b, dump_h;
  // work-item counters (the DUMP variant does not use them): zero at launch,
  // left zero by a launch that runs to its end
  uint32_t* sched;
  int sched_s0;                // items of an XCD range taken by static index (set by launch_attention)
  int sched_n_claim;           // workgroups that claim the rest (0: all static)
};

hipError_t launch_prepare(const PrepArgs& a, bool fp16, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, bool repair, bool dump, hipStream_t st);

}  // namespace oc
