// Host side of liboc_attn.so: the C ABI declared in include/oc_attn.h.
// Validation happens before any HIP call, so every argument error is
// reported the same way with or without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/oc_attn.h"
#include "oc_common.h"
#include "oc_kernels.h"

using namespace oc;

namespace {

thread_local int g_last_hip_error = 0;

oc_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return OC_ERR_HIP;
}

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

int repair_count(double budget, int S) {
  // ceil(budget * S) with a 1e-9 allowance for binary rounding, capped at S
  if (!(budget > 0.0)) return 0;
  const double k = std::ceil(budget * (double)S - 1e-9);
  if (k <= 0.0) return 0;
  return k >= (double)S ? S : (int)k;
}

bool env_flag(const char* name) {
  const char* s = std::getenv(name);
  return s && *s && std::strcmp(s, "0") != 0;
}

}  // namespace

struct oc_attn_plan {
  oc_attn_desc d;
  double max_budget;
  float tau;
  int n_sel_max;
  oc_attn_ws_layout L;
  int order;
  int exp_path;          // oc_weights: 0 ExpCast, 1 exp + FP8 cast
  int k_smooth;          // K-mean smoothing in prepare
  int v_smooth;          // V-Smooth block means (prepare and attention)
  // cached prepare graph
  hipGraphExec_t gexec = nullptr;
  hipStream_t cap_stream = nullptr;
  const void *gq = nullptr, *gk = nullptr, *gv = nullptr;
  void* gws = nullptr;
  int gnsel = -1;
  int gksmooth = -1;
  int gvsmooth = -1;
  // the workspaces this plan prepared most recently, with their repair count
  // (-1: prepared without repair)
  static constexpr int NPREP = 64;
  const void* prepared_ws[NPREP] = {};
  int prepared_nsel[NPREP] = {};
  int prepared_vs[NPREP] = {};
  int prepared_next = 0;

  void mark_prepared(const void* ws, int nsel, int vs) {
    for (int i = 0; i < NPREP; ++i)
      if (prepared_ws[i] == ws) {
        prepared_nsel[i] = nsel;
        prepared_vs[i] = vs;
        return;
      }
    prepared_ws[prepared_next] = ws;
    prepared_nsel[prepared_next] = nsel;
    prepared_vs[prepared_next] = vs;
    prepared_next = (prepared_next + 1) % NPREP;
  }
  // repair count the workspace was prepared with; -2 if this plan never prepared it
  int prepared_state(const void* ws) const {
    for (int i = 0; i < NPREP; ++i)
      if (prepared_ws[i] == ws) return prepared_nsel[i];
    return -2;
  }
  // whether the workspace holds V-Smooth residuals (the attention kernel must
  // then add the block means back)
  int prepared_vsmooth(const void* ws) const {
    for (int i = 0; i < NPREP; ++i)
      if (prepared_ws[i] == ws) return prepared_vs[i];
    return 0;
  }
};

static void compute_layout(oc_attn_plan* p) {
  const oc_attn_desc& d = p->d;
  const uint64_t BH = (uint64_t)d.B * d.H;
  oc_attn_ws_layout& L = p->L;
  std::memset(&L, 0, sizeof(L));
  L.n_ktiles = (d.S + KTILE - 1) / KTILE;
  L.n_qtiles = (d.S + BQ - 1) / BQ;
  L.s_pad_q = L.n_qtiles * BQ;
  L.n_sel_max = p->n_sel_max;
  L.n_sel_tiles_max = (p->n_sel_max + KTILE - 1) / KTILE;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.qhat = take(BH * L.s_pad_q * HEAD_DIM);
  L.kpack = take(BH * L.n_ktiles * (uint64_t)TILE_BYTES);
  L.vpack = take(BH * L.n_ktiles * (uint64_t)TILE_BYTES);
  L.sq = take(BH * (L.s_pad_q / KTILE) * 4);
  L.sk = take(BH * L.n_ktiles * 4);
  L.vamax = take(BH * L.n_ktiles * 4);
  L.sv = take(BH * 2 * 4);
  if (p->n_sel_max > 0) {
    L.energy = take(BH * (uint64_t)d.S * 8);
    L.sel = take(BH * (uint64_t)p->n_sel_max * 4);
    L.kselpack = take(BH * L.n_sel_tiles_max * (uint64_t)TILE_BYTES);
    L.rpack = take(BH * L.n_sel_tiles_max * (uint64_t)TILE_BYTES);
    L.sksel = take(BH * L.n_sel_tiles_max * (uint64_t)KTILE * 4);
    L.sr = take(BH * 2 * 4);
  }
  L.kmean = take(BH * HEAD_DIM * 4);
  L.kpart = take(BH * L.n_ktiles * (uint64_t)HEAD_DIM * 8);
  L.vmu = take(BH * L.n_ktiles * (uint64_t)HEAD_DIM * 2);
  L.sched = take(SCHED_WORDS * 4);
  L.total_bytes = off;
}

static bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

static uint64_t input_extent_bytes(const oc_attn_desc& d) {
  return 2ull * ((uint64_t)(d.B - 1) * d.stride_b + (uint64_t)(d.S - 1) * d.stride_s +
                 (uint64_t)(d.H - 1) * d.stride_h + HEAD_DIM);
}

static bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static oc_status check_inputs(const oc_attn_plan* p, const void* q, const void* k, const void* v, const void* ws,
                              size_t ws_bytes) {
  if (!q || !k || !v || !ws) return OC_ERR_INVALID_ARGUMENT;
  if (misaligned(q) || misaligned(k) || misaligned(v) || ((uintptr_t)ws & 255u)) return OC_ERR_INVALID_ARGUMENT;
  if (ws_bytes < p->L.total_bytes) return OC_ERR_WORKSPACE_TOO_SMALL;
  const uint64_t ext = input_extent_bytes(p->d);
  if (overlap(ws, ws_bytes, q, ext) || overlap(ws, ws_bytes, k, ext) || overlap(ws, ws_bytes, v, ext))
    return OC_ERR_INVALID_ARGUMENT;
  return OC_OK;
}

static oc_status check_out(const oc_attn_plan* p, const void* out, const void* const* others, int n_others,
                           const void* ws, size_t ws_bytes) {
  if (!out || misaligned(out)) return OC_ERR_INVALID_ARGUMENT;
  const uint64_t on = 2ull * p->d.B * p->d.S * p->d.H * HEAD_DIM;
  const uint64_t ext = input_extent_bytes(p->d);
  for (int i = 0; i < n_others; ++i)
    if (others[i] && overlap(out, on, others[i], ext)) return OC_ERR_INVALID_ARGUMENT;
  if (overlap(out, on, ws, ws_bytes)) return OC_ERR_INVALID_ARGUMENT;
  return OC_OK;
}

static oc_status check_budget(const oc_attn_plan* p, double budget) {
  if (!(budget >= 0.0) || !(budget <= 1.0) || std::isnan(budget)) return OC_ERR_INVALID_ARGUMENT;
  if (repair_count(budget, p->d.S) > p->n_sel_max) return OC_ERR_INVALID_ARGUMENT;
  return OC_OK;
}

static PrepArgs prep_args(const oc_attn_plan* p, const void* q, const void* k, const void* v, void* ws, int n_sel) {
  const oc_attn_desc& d = p->d;
  const oc_attn_ws_layout& L = p->L;
  uint8_t* base = (uint8_t*)ws;
  PrepArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.sb = d.stride_b;
  a.ss = d.stride_s;
  a.sh = d.stride_h;
  a.B = d.B;
  a.S = d.S;
  a.H = d.H;
  a.nT = L.n_ktiles;
  a.nQB = L.s_pad_q / KTILE;
  a.s_pad_q = L.s_pad_q;
  a.qhat = base + L.qhat;
  a.kpack = base + L.kpack;
  a.vpack = base + L.vpack;
  a.sq = (float*)(base + L.sq);
  a.sk = (float*)(base + L.sk);
  a.vamax = (float*)(base + L.vamax);
  a.sv = (float*)(base + L.sv);
  a.sched = (uint32_t*)(base + L.sched);
  if (p->k_smooth) {
    a.kmean = (float*)(base + L.kmean);
    a.kpart = (double*)(base + L.kpart);
  }
  if (p->v_smooth) {
    a.vmu = (uint16_t*)(base + L.vmu);
  }
  if (n_sel > 0) {
    a.energy = (double*)(base + L.energy);
    a.sel = (int32_t*)(base + L.sel);
    a.kselpack = base + L.kselpack;
    a.rpack = base + L.rpack;
    a.sksel = (float*)(base + L.sksel);
    a.sr = (float*)(base + L.sr);
    a.n_sel = n_sel;
    a.n_sel_tiles = (n_sel + KTILE - 1) / KTILE;
  }
  return a;
}

static AttnArgs attn_args(const oc_attn_plan* p, const void* ws, void* out, int n_sel) {
  const oc_attn_desc& d = p->d;
  const oc_attn_ws_layout& L = p->L;
  const uint8_t* base = (const uint8_t*)ws;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.qhat = base + L.qhat;
  a.kpack = base + L.kpack;
  a.vpack = base + L.vpack;
  a.sq = (const float*)(base + L.sq);
  a.sk = (const float*)(base + L.sk);
  a.sv = (const float*)(base + L.sv);
  if (n_sel > 0) {
    a.kselpack = base + L.kselpack;
    a.rpack = base + L.rpack;
    a.sksel = (const float*)(base + L.sksel);
    a.sr = (const float*)(base + L.sr);
    a.n_sel = n_sel;
    a.n_sel_tiles = (n_sel + KTILE - 1) / KTILE;
  }
  a.out = (uint16_t*)out;
  a.B = d.B;
  a.S = d.S;
  a.H = d.H;
  a.nT = L.n_ktiles;
  a.nQT = L.n_qtiles;
  a.nQB = L.s_pad_q / KTILE;
  a.s_pad_q = L.s_pad_q;
  a.c8 = (float)(8.0 * (double)p->tau * 1.4426950408889634);
  a.order = p->order;
  a.exp_path = p->exp_path;
  a.vmu = p->prepared_vsmooth(ws) ? (const uint16_t*)(base + L.vmu) : nullptr;
  return a;
}

// Enqueue the prepare kernels: directly, or with OC_ATTN_GRAPH=1 in the
// environment through the plan's cached graph (captured once per set of
// pointers and options, then replayed). Launching the two to five kernels
// directly costs less on this platform: a graph launch adds about 15 us of
// GPU time, which on short sequences is as much as the kernels themselves.
// n_sel < 0: plain prepare; n_sel >= 0: prepare for repair with that many
// selected tokens (0 selects none).
static oc_status run_prepare(oc_attn_plan* p, const void* q, const void* k, const void* v, void* ws, int n_sel,
                             hipStream_t st) {
  const PrepArgs a = prep_args(p, q, k, v, ws, n_sel);
  const bool fp16 = p->d.dtype == OC_FP16;
  hipError_t e;
  if (!env_flag("OC_ATTN_GRAPH")) {
    e = launch_prepare(a, fp16, st);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    if (!(p->gexec && p->gq == q && p->gk == k && p->gv == v && p->gws == ws && p->gnsel == n_sel &&
          p->gksmooth == p->k_smooth && p->gvsmooth == p->v_smooth)) {
      if (p->gexec) {
        (void)hipGraphExecDestroy(p->gexec);
        p->gexec = nullptr;
      }
      if (!p->cap_stream) {
        e = hipStreamCreateWithFlags(&p->cap_stream, hipStreamNonBlocking);
        if (e != hipSuccess) return hip_fail(e);
      }
      e = hipStreamBeginCapture(p->cap_stream, hipStreamCaptureModeThreadLocal);
      if (e != hipSuccess) return hip_fail(e);
      const hipError_t le = launch_prepare(a, fp16, p->cap_stream);
      hipGraph_t graph = nullptr;
      e = hipStreamEndCapture(p->cap_stream, &graph);
      if (le != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return hip_fail(le);
      }
      if (e != hipSuccess) return hip_fail(e);
      e = hipGraphInstantiate(&p->gexec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (e != hipSuccess) {
        p->gexec = nullptr;
        return hip_fail(e);
      }
      p->gq = q;
      p->gk = k;
      p->gv = v;
      p->gws = ws;
      p->gnsel = n_sel;
      p->gksmooth = p->k_smooth;
      p->gvsmooth = p->v_smooth;
    }
    e = hipGraphLaunch(p->gexec, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  p->mark_prepared(ws, n_sel, p->v_smooth);
  return OC_OK;
}

static oc_status run_attention(oc_attn_plan* p, void* ws, void* out, int n_sel, hipStream_t st) {
  AttnArgs a = attn_args(p, ws, out, n_sel);
  a.sched = (uint32_t*)((uint8_t*)ws + p->L.sched);
  const hipError_t e = launch_attention(a, n_sel > 0, false, st);
  return e == hipSuccess ? OC_OK : hip_fail(e);
}

// Workspace of oc_attn_forward_v_repair_noalloc: a file-scope device array,
// one copy per GPU, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol):
// it looks up each device's own address once, with that device current,
// and passes that.
static __device__ __align__(256) uint8_t scratch[OC_NOALLOC_WORKSPACE_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// device address of the current device's scratch array (looked up on the
// first call on each device)
oc_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= MAX_DEVICES) return OC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return OC_OK;
}
// One line per C-ABI call on stderr when the environment sets OC_ATTN_LOG=1
// (read once): the entry point, the plan's shape and options, the budget of
// the repair calls, and the status (with the HIP error for OC_ERR_HIP).
bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("OC_ATTN_LOG");
    return e != nullptr && std::atoi(e) == 1;
  }();
  return on;
}

oc_status logged(const char* fn, const oc_attn_plan* p, oc_status s, double budget,
                 const oc_attn_desc* desc = nullptr) {
  if (!log_enabled()) return s;
  char line[512];
  int n = std::snprintf(line, sizeof line, "[oc_attn] %s", fn);
  const oc_attn_desc* d = p ? &p->d : desc;
  if (d && n > 0 && n < (int)sizeof line)
    n += std::snprintf(line + n, sizeof line - n, " B=%d S=%d H=%d D=%d %s", d->B, d->S, d->H, d->D,
                       d->dtype == OC_FP16 ? "fp16" : "bf16");
  if (p && n > 0 && n < (int)sizeof line)
    n += std::snprintf(line + n, sizeof line - n, " weights=%s v_smooth=%d k_smooth=%d",
                       p->exp_path ? "exp_fp8" : "expcast", p->v_smooth, p->k_smooth);
  if (budget >= 0.0 && n > 0 && n < (int)sizeof line)
    n += std::snprintf(line + n, sizeof line - n, " budget=%g", budget);
  if (n > 0 && n < (int)sizeof line)
    n += std::snprintf(line + n, sizeof line - n, " -> %s", oc_attn_status_string(s));
  if (s == OC_ERR_HIP && n > 0 && n < (int)sizeof line)
    n += std::snprintf(line + n, sizeof line - n, " (%s)", hipGetErrorString((hipError_t)g_last_hip_error));
  std::fprintf(stderr, "%s\n", line);
  return s;
}
}  // namespace

extern "C" {

static oc_status plan_create_impl(const oc_attn_desc* desc, double max_repair_budget, oc_attn_plan** plan) {
  if (!desc || !plan) return OC_ERR_INVALID_ARGUMENT;
  *plan = nullptr;
  const oc_attn_desc& d = *desc;
  if (d.D != HEAD_DIM) return OC_ERR_UNSUPPORTED;
  if (d.dtype != OC_BF16 && d.dtype != OC_FP16) return OC_ERR_UNSUPPORTED;
  if (d.B < 1 || d.S < 1 || d.H < 1) return OC_ERR_INVALID_ARGUMENT;
  if (d.stride_b < 0 || d.stride_s < 0 || d.stride_h < 0) return OC_ERR_INVALID_ARGUMENT;
  // 16-byte rows: every stride a multiple of 8 elements
  if ((d.stride_b | d.stride_s | d.stride_h) & 7) return OC_ERR_INVALID_ARGUMENT;
  if (!(d.softmax_scale >= 0.0f) || std::isinf(d.softmax_scale)) return OC_ERR_INVALID_ARGUMENT;
  if (!(max_repair_budget >= 0.0 && max_repair_budget <= 1.0)) return OC_ERR_INVALID_ARGUMENT;
  // index arithmetic in the kernels uses 32-bit tile and row counts
  if ((int64_t)d.B * d.H * (((int64_t)d.S + BQ - 1) / BQ) > (int64_t)INT32_MAX / 8) return OC_ERR_UNSUPPORTED;
  oc_attn_plan* p = new (std::nothrow) oc_attn_plan();
  if (!p) return OC_ERR_INVALID_ARGUMENT;
  p->d = d;
  p->max_budget = max_repair_budget;
  p->tau = d.softmax_scale > 0.0f ? d.softmax_scale : (float)(1.0 / std::sqrt((double)d.D));
  p->n_sel_max = repair_count(max_repair_budget, d.S);
  const char* order = std::getenv("OC_ATTN_ORDER");
  p->order = (order && std::atoi(order) == 1) ? 1 : 0;
  compute_layout(p);
  *plan = p;
  return OC_OK;
}

static oc_status plan_set_weights_impl(oc_attn_plan* p, int weights) {
  if (!p || (weights != OC_WEIGHTS_EXPCAST && weights != OC_WEIGHTS_EXP_FP8)) return OC_ERR_INVALID_ARGUMENT;
  p->exp_path = weights == OC_WEIGHTS_EXP_FP8 ? 1 : 0;
  return OC_OK;
}

static oc_status plan_set_v_smoothing_impl(oc_attn_plan* p, int enable) {
  if (!p || (enable != 0 && enable != 1)) return OC_ERR_INVALID_ARGUMENT;
  p->v_smooth = enable;
  return OC_OK;
}

static oc_status plan_set_k_smoothing_impl(oc_attn_plan* p, int enable) {
  if (!p || (enable != 0 && enable != 1)) return OC_ERR_INVALID_ARGUMENT;
  p->k_smooth = enable;
  return OC_OK;
}

void oc_attn_plan_destroy(oc_attn_plan* p) {
  if (!p) return;
  if (p->gexec) (void)hipGraphExecDestroy(p->gexec);
  if (p->cap_stream) (void)hipStreamDestroy(p->cap_stream);
  delete p;
}

static oc_status workspace_size_impl(const oc_attn_plan* p, size_t* bytes) {
  if (!p || !bytes) return OC_ERR_INVALID_ARGUMENT;
  *bytes = (size_t)p->L.total_bytes;
  return OC_OK;
}

static oc_status workspace_layout_impl(const oc_attn_plan* p, oc_attn_ws_layout* layout) {
  if (!p || !layout) return OC_ERR_INVALID_ARGUMENT;
  *layout = p->L;
  return OC_OK;
}

static oc_status prepare_impl(oc_attn_plan* p, const void* q, const void* k, const void* v, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!p) return OC_ERR_INVALID_ARGUMENT;
  oc_status s = check_inputs(p, q, k, v, ws, ws_bytes);
  if (s != OC_OK) return s;
  return run_prepare(p, q, k, v, ws, -1, (hipStream_t)stream);
}

static oc_status forward_impl(oc_attn_plan* p, const void* q, const void* k, const void* v, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!p) return OC_ERR_INVALID_ARGUMENT;
  oc_status s = check_inputs(p, q, k, v, ws, ws_bytes);
  if (s != OC_OK) return s;
  const void* ins[3] = {q, k, v};
  s = check_out(p, out, ins, 3, ws, ws_bytes);
  if (s != OC_OK) return s;
  s = run_prepare(p, q, k, v, ws, -1, (hipStream_t)stream);
  if (s != OC_OK) return s;
  return run_attention(p, ws, out, 0, (hipStream_t)stream);
}

static oc_status prepare_v_repair_impl(oc_attn_plan* p, const void* q, const void* k, const void* v, double budget,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!p) return OC_ERR_INVALID_ARGUMENT;
  oc_status s = check_budget(p, budget);
  if (s != OC_OK) return s;
  s = check_inputs(p, q, k, v, ws, ws_bytes);
  if (s != OC_OK) return s;
  return run_prepare(p, q, k, v, ws, repair_count(budget, p->d.S), (hipStream_t)stream);
}

static oc_status forward_v_repair_impl(oc_attn_plan* p, const void* q, const void* k, const void* v, double budget,
                                   void* out, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return OC_ERR_INVALID_ARGUMENT;
  oc_status s = check_budget(p, budget);
  if (s != OC_OK) return s;
  s = check_inputs(p, q, k, v, ws, ws_bytes);
  if (s != OC_OK) return s;
  const void* ins[3] = {q, k, v};
  s = check_out(p, out, ins, 3, ws, ws_bytes);
  if (s != OC_OK) return s;
  const int n_sel = repair_count(budget, p->d.S);
  s = run_prepare(p, q, k, v, ws, n_sel, (hipStream_t)stream);
  if (s != OC_OK) return s;
  return run_attention(p, ws, out, n_sel, (hipStream_t)stream);
}

static oc_status forward_v_repair_noalloc_impl(oc_attn_plan* p, const void* q, const void* k, const void* v,
                                          double budget, void* out, void* stream) {
  if (!p) return OC_ERR_INVALID_ARGUMENT;
  if (p->L.total_bytes > OC_NOALLOC_WORKSPACE_BYTES) return OC_ERR_WORKSPACE_TOO_SMALL;
  oc_status s = check_budget(p, budget);
  if (s != OC_OK) return s;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != OC_OK) return s;
  const size_t ws_bytes = OC_NOALLOC_WORKSPACE_BYTES;
  s = check_inputs(p, q, k, v, ws, ws_bytes);
  if (s != OC_OK) return s;
  const void* ins[3] = {q, k, v};
  s = check_out(p, out, ins, 3, ws, ws_bytes);
  if (s != OC_OK) return s;
  // the kernels one by one: no graph is captured or instantiated here
  const int n_sel = repair_count(budget, p->d.S);
  const hipError_t e = launch_prepare(prep_args(p, q, k, v, ws, n_sel > 0 ? n_sel : -1), p->d.dtype == OC_FP16,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  p->mark_prepared(ws, n_sel > 0 ? n_sel : -1, p->v_smooth);
  return run_attention(p, ws, out, n_sel, (hipStream_t)stream);
}

static oc_status forward_prepared_impl(oc_attn_plan* p, void* ws, size_t ws_bytes, void* out, int with_repair,
                                   void* stream) {
  if (!p || !ws || ((uintptr_t)ws & 255u)) return OC_ERR_INVALID_ARGUMENT;
  if (ws_bytes < p->L.total_bytes) return OC_ERR_WORKSPACE_TOO_SMALL;
  oc_status s = check_out(p, out, nullptr, 0, ws, ws_bytes);
  if (s != OC_OK) return s;
  const int state = p->prepared_state(ws);
  if (state == -2) return OC_ERR_NOT_PREPARED;
  if (with_repair && state < 0) return OC_ERR_NOT_PREPARED;
  return run_attention(p, ws, out, with_repair ? state : 0, (hipStream_t)stream);
}

static oc_status debug_pcodes_impl(oc_attn_plan* p, const void* ws, size_t ws_bytes, int32_t b, int32_t h,
                               const int32_t* rows, int32_t n_rows, int32_t with_repair, uint8_t* codes,
                               int32_t* m_used, float* scores, uint8_t* rcodes, float* out_f32, void* out,
                               void* stream) {
  if (!p || !ws || !out || !rows || ((uintptr_t)ws & 255u)) return OC_ERR_INVALID_ARGUMENT;
  if (b < 0 || b >= p->d.B || h < 0 || h >= p->d.H) return OC_ERR_INVALID_ARGUMENT;
  if (n_rows < 1 || n_rows > p->d.S) return OC_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)rows & 3u) || ((uintptr_t)m_used & 3u) || ((uintptr_t)scores & 3u) || ((uintptr_t)out_f32 & 15u))
    return OC_ERR_INVALID_ARGUMENT;
  if (ws_bytes < p->L.total_bytes) return OC_ERR_WORKSPACE_TOO_SMALL;
  oc_status s = check_out(p, out, nullptr, 0, ws, ws_bytes);
  if (s != OC_OK) return s;
  const int state = p->prepared_state(ws);
  if (state == -2) return OC_ERR_NOT_PREPARED;
  if (with_repair && state < 0) return OC_ERR_NOT_PREPARED;
  const int n_sel = with_repair ? state : 0;
  AttnArgs a = attn_args(p, ws, out, n_sel);
  a.dump_rows = rows;
  a.n_dump = n_rows;
  a.dump_codes = codes;
  a.dump_m = m_used;
  a.dump_scores = scores;
  a.dump_rcodes = n_sel > 0 ? rcodes : nullptr;
  a.dump_out32 = out_f32;
  a.dump_b = b;
  a.dump_h = h;
  const hipError_t e = launch_attention(a, n_sel > 0, true, (hipStream_t)stream);
  return e == hipSuccess ? OC_OK : hip_fail(e);
}

const char* oc_attn_status_string(oc_status s) {
  switch (s) {
    case OC_OK: return "ok";
    case OC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case OC_ERR_UNSUPPORTED: return "unsupported (D must be 128; dtype bf16 or fp16)";
    case OC_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case OC_ERR_NOT_PREPARED: return "workspace not prepared by this plan";
    case OC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int oc_attn_last_hip_error(void) { return g_last_hip_error; }


oc_status oc_attn_plan_create(const oc_attn_desc* desc, double max_repair_budget, oc_attn_plan** plan) {
  const oc_status s = plan_create_impl(desc, max_repair_budget, plan);
  return logged("oc_attn_plan_create", s == OC_OK ? *plan : nullptr, s, max_repair_budget, desc);
}

oc_status oc_attn_plan_set_weights(oc_attn_plan* p, int weights) {
  return logged("oc_attn_plan_set_weights", p, plan_set_weights_impl(p, weights), -1.0);
}

oc_status oc_attn_plan_set_v_smoothing(oc_attn_plan* p, int enable) {
  return logged("oc_attn_plan_set_v_smoothing", p, plan_set_v_smoothing_impl(p, enable), -1.0);
}

oc_status oc_attn_plan_set_k_smoothing(oc_attn_plan* p, int enable) {
  return logged("oc_attn_plan_set_k_smoothing", p, plan_set_k_smoothing_impl(p, enable), -1.0);
}

oc_status oc_attn_workspace_size(const oc_attn_plan* p, size_t* bytes) {
  return logged("oc_attn_workspace_size", p, workspace_size_impl(p, bytes), -1.0);
}

oc_status oc_attn_workspace_layout(const oc_attn_plan* p, oc_attn_ws_layout* layout) {
  return logged("oc_attn_workspace_layout", p, workspace_layout_impl(p, layout), -1.0);
}

oc_status oc_attn_prepare(oc_attn_plan* p, const void* q, const void* k, const void* v, void* ws, size_t ws_bytes,
                          void* stream) {
  return logged("oc_attn_prepare", p, prepare_impl(p, q, k, v, ws, ws_bytes, stream), -1.0);
}

oc_status oc_attn_forward(oc_attn_plan* p, const void* q, const void* k, const void* v, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
  return logged("oc_attn_forward", p, forward_impl(p, q, k, v, out, ws, ws_bytes, stream), -1.0);
}

oc_status oc_attn_prepare_v_repair(oc_attn_plan* p, const void* q, const void* k, const void* v, double budget,
                                   void* ws, size_t ws_bytes, void* stream) {
  return logged("oc_attn_prepare_v_repair", p, prepare_v_repair_impl(p, q, k, v, budget, ws, ws_bytes, stream), budget);
}

oc_status oc_attn_forward_v_repair(oc_attn_plan* p, const void* q, const void* k, const void* v, double budget,
                                   void* out, void* ws, size_t ws_bytes, void* stream) {
  return logged("oc_attn_forward_v_repair", p, forward_v_repair_impl(p, q, k, v, budget, out, ws, ws_bytes, stream), budget);
}

oc_status oc_attn_forward_v_repair_noalloc(oc_attn_plan* p, const void* q, const void* k, const void* v,
                                          double budget, void* out, void* stream) {
  return logged("oc_attn_forward_v_repair_noalloc", p, forward_v_repair_noalloc_impl(p, q, k, v, budget, out, stream), budget);
}

oc_status oc_attn_forward_prepared(oc_attn_plan* p, void* ws, size_t ws_bytes, void* out, int with_repair,
                                   void* stream) {
  return logged("oc_attn_forward_prepared", p, forward_prepared_impl(p, ws, ws_bytes, out, with_repair, stream), -1.0);
}

oc_status oc_attn_debug_pcodes(oc_attn_plan* p, const void* ws, size_t ws_bytes, int32_t b, int32_t h,
                               const int32_t* rows, int32_t n_rows, int32_t with_repair, uint8_t* codes,
                               int32_t* m_used, float* scores, uint8_t* rcodes, float* out_f32, void* out,
                               void* stream) {
  return logged("oc_attn_debug_pcodes", p, debug_pcodes_impl(p, ws, ws_bytes, b, h, rows, n_rows, with_repair, codes, m_used, scores, rcodes, out_f32, out, stream), -1.0);
}

}  // extern "C"
