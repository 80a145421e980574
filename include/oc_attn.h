/*
 * oc_attn — ExpCast FP8 forward attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of liboc_attn.so. Plain pointers and sizes only.
 *
 * What the library computes (sources are the pages on Open-VC Attention and
 * VC-Attention):
 *   - Open VC Attention product page (ailibri.com), API paragraph:
 *     non-causal multi-head forward attention with head dimension 128 on
 *     FP16 or BF16 inputs laid out [B,S,H,128] (or [S,H,128]). The call
 *     quantizes to FP8 itself, runs ExpCast attention, and returns BF16.
 *   - same page, kernel paragraph: softmax weights go to FP8 straight from
 *     the scores. Q and K carry per-block scales and V a per-head scale.
 *     Key tiles are visited starting from the middle of the window.
 *   - VC-Attention write-up (Nunchux AI), section "ExpCast-FP8": the FP8 byte
 *     of a weight is produced from the log-domain score with one fused
 *     multiply-add (E4M3 byte as integer ~ 8*log2(v) + 56, beta = -0.35),
 *     with no exponential and no FP32->FP8 conversion.
 *   - Open-VC news (aikraft.ru), sections "Решение: ExpCast и отказ от
 *     экспонент" (V-residual repair of the worst-rounded value tokens) and
 *     "Архитектурные оптимизации" (mid-window traversal; Q/K/V preparation
 *     fused into one graph); product page, repair paragraph (prepare with a
 *     budget such as 0.005, then the repaired attention call).
 *
 * Per (b, h), with tau the softmax scale:
 *   Q/K: per 128-token block, s = amax/448 (fp32). The code is E4M3(q * 448/amax),
 *        round to nearest even, saturating.
 *   V:   one scale per head, sv = amax/448, same rounding.
 *   A block, head or repair set whose amax is below 2^-100 (an all-zero one
 *   included) takes s = 1: every code is then 0 and those values count as 0.
 *   x_ij  = tau*log2(e) * sq_i * sk_j * <q_hat_i, k_hat_j>
 *   M_i   = ceil(max_j x_ij)                      (bit-aligned row max)
 *   c_ij  = clamp(rne(8*(x_ij - M_i) + 119.65), 0, 126)   (E4M3 byte of 256*2^(x-M))
 *   L_i   = sum_j dec(c_ij)
 *   O_i   = sv * sum_j dec(c_ij) v_hat_j / L_i    -> BF16
 *   repair (budget b): the k = ceil(b*S) tokens with the largest residual
 *   energy sum_c (v - sv*dec(v_hat))^2 get sr * dec(r_hat_j) added to their
 *   value. r_hat is the E4M3 residual with its own per-head scale sr. L is
 *   left unchanged.
 *
 * Layout: q, k and v are [B,S,H,128] with element strides (stride_b,
 * stride_s, stride_h) shared by the three tensors; the channel stride is 1.
 * `out` is a contiguous BF16 [B,S,H,128] tensor. q, k, v and out must be
 * 16-byte aligned and every stride a multiple of 8 elements; the workspace
 * must be 256-byte aligned.
 *
 * Ownership: the caller allocates and owns q, k, v, out and the workspace
 * (device memory). The library never allocates or frees device memory in
 * these calls. A plan owns only host state: the descriptor, its sizes, and,
 * when OC_ATTN_GRAPH=1 is set, a cached hipGraphExec of the prepare step,
 * keyed on the pointers it was captured with. A plan is used from one host
 * thread at a time.
 *
 * Execution: every call enqueues work on `stream` (a hipStream_t; NULL is the
 * default stream) and returns without synchronizing. Inputs are never
 * modified. `out` must not overlap q, k, v or the workspace. Every call that
 * takes a writable workspace writes to it, oc_attn_forward_prepared included
 * (the attention kernel claims work items through counters kept there), so
 * calls that share a workspace must not overlap: enqueue them on one stream,
 * or order their streams.
 *
 * Errors: every call returns an oc_status. Arguments are validated before
 * anything is enqueued:
 *   - D != 128 or an unknown dtype gives OC_ERR_UNSUPPORTED;
 *   - B, S or H < 1, a NULL or misaligned pointer, a negative stride, a
 *     budget outside [0, max budget of the plan] or NaN, or overlapping
 *     buffers give OC_ERR_INVALID_ARGUMENT;
 *   - a workspace smaller than oc_attn_workspace_size gives
 *     OC_ERR_WORKSPACE_TOO_SMALL;
 *   - oc_attn_forward_prepared on a workspace this plan has not prepared
 *     (or, with repair, not prepared with repair) gives OC_ERR_NOT_PREPARED.
 *   A failing HIP call gives OC_ERR_HIP. oc_attn_last_hip_error() then
 *   returns the hipError_t of the calling thread's last failure.
 *
 * Logging: with OC_ATTN_LOG=1 in the environment (read once per process),
 * every call above writes one line to stderr: the entry point, the plan's
 * B, S, H, D, dtype and options, the budget of the repair calls, and the
 * status (with the HIP error's text for OC_ERR_HIP). Otherwise the library
 * prints nothing.
 * NaN or Inf inputs are not supported; the output for them is undefined.
 * Otherwise the output is finite wherever the method's own result is, with
 * one exception in the V-Smooth option (oc_attn_plan_set_v_smoothing): when
 * a head's block means exceed its smoothed residuals by more than about
 * 2^60 (for example means near 1e20 beside residuals near 1e-25), the mean
 * term can overflow the fp32 accumulator.
 */
#ifndef OC_ATTN_H
#define OC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum oc_status {
  OC_OK = 0,
  OC_ERR_INVALID_ARGUMENT = 1,
  OC_ERR_UNSUPPORTED = 2,
  OC_ERR_WORKSPACE_TOO_SMALL = 3,
  OC_ERR_NOT_PREPARED = 4,
  OC_ERR_HIP = 5
} oc_status;

typedef enum oc_dtype { OC_BF16 = 0, OC_FP16 = 1 } oc_dtype;

typedef struct oc_attn_desc {
  int32_t B, S, H, D;          /* batch, sequence length, heads, head dim (must be 128) */
  int32_t dtype;               /* oc_dtype of q, k and v */
  int64_t stride_b;            /* element strides of q, k, v; channel stride is 1 */
  int64_t stride_s;
  int64_t stride_h;
  float softmax_scale;         /* tau; 0 selects 1/sqrt(D) */
} oc_attn_desc;

/* Byte offsets of the buffers inside a workspace (all 256-byte aligned), and
 * the tile counts. Exposed so that tests can read the prepared FP8 tensors. Layouts:
 *   qhat   u8  [B][H][s_pad_q][128]        natural order, padding rows 0
 *   kpack  u8  [B][H][n_ktiles][16384]     key tiles of 128 keys x 128 channels
 *                                          in MFMA operand order: columns
 *                                          32g+16h..+16 of row r (g, h in
 *                                          0..3, 0..1) form 16-byte chunk
 *                                          (2*(r/16) + h)*64 + 16g + r%16
 *   vpack  u8  [B][H][n_ktiles][16384]     transposed value tiles (rows =
 *                                          channels d, columns = keys), same
 *                                          chunk order; key j of the tile sits
 *                                          at column kk = 32*((j>>2)&3) + 4*(j>>4) + (j&3)
 *   sq     f32 [B][H][s_pad_q/128]    sk, vamax f32 [B][H][n_ktiles]
 *   sv     f32 [B][H][2]              {amax/448, 448/amax} of the head's V
 *   energy f64 [B][H][S]              residual energy (repair only)
 *   sel    i32 [B][H][n_sel]          selected tokens, ascending
 *   kselpack, rpack: like kpack/vpack over the selected tokens (slot order),
 *                                     [B][H][n_sel_tiles][128][128]
 *   sksel  f32 [B][H][n_sel_tiles*128]  K block scale of each selected token
 *   (the repair buffers are packed with the n_sel = ceil(budget*S) and
 *    n_sel_tiles = ceil(n_sel/128) of the last prepare_v_repair, inside
 *    space sized for the plan's maximum budget)
 *   sr     f32 [B][H][2]              {amax/448, 448/amax} of the selected residuals
 *   kmean  f32 [B][H][128]            mean key per channel (K-mean smoothing only)
 *   kpart  f64 [B][H][n_ktiles][128]  per-block key sums (K-mean smoothing only)
 *   vmu    bf16 [B][H][n_ktiles][128] V block means (V-Smooth only; vpack then
 *                                     holds the codes of v - mean, and sv and
 *                                     vamax refer to those residuals)
 *   sched  u32 [16]                   work-item counters of the attention
 *                                     kernel on long inputs (at least 4096
 *                                     (b, h, 256-query tile) items): every
 *                                     prepare call zeroes them, and every
 *                                     attention launch that runs to its end
 *                                     leaves them zero again
 */
typedef struct oc_attn_ws_layout {
  uint64_t qhat, kpack, vpack, sq, sk, vamax, sv;
  uint64_t energy, sel, kselpack, rpack, sksel, sr;
  uint64_t kmean, kpart, vmu, sched;
  uint64_t total_bytes;
  int32_t n_ktiles, n_qtiles, s_pad_q, n_sel_max, n_sel_tiles_max;
} oc_attn_ws_layout;

typedef struct oc_attn_plan oc_attn_plan;

/* Create a plan for one problem shape. max_repair_budget in [0, 1] sizes the
 * repair buffers (0 = no repair). Host-only; makes no HIP call. */
oc_status oc_attn_plan_create(const oc_attn_desc* desc, double max_repair_budget, oc_attn_plan** plan);
/* Release a plan (and its cached graph). NULL is ignored. */
void oc_attn_plan_destroy(oc_attn_plan* plan);
/* Softmax-weight path of the attention kernel, for later oc_attn_forward*,
 * oc_attn_forward_prepared and oc_attn_debug_pcodes calls on this plan
 * (host-only; default OC_WEIGHTS_EXPCAST).
 *   OC_WEIGHTS_EXPCAST: E4M3 bytes from one FMA on the log-domain score
 *     (VC-Attention write-up, section "ExpCast-FP8").
 *   OC_WEIGHTS_EXP_FP8: the path ExpCast replaces, kept to measure what it
 *     saves (Open-VC news, section "Проблема: узкое место MUFU в FP8": one
 *     exponential per score; VC-Attention write-up, section "ExpCast-FP8":
 *     exponential, then an FP32->FP8 cast). Weight 256*2^(x - M) from one
 *     v_exp_f32 per score (within 1 ulp of the rounded value), then the
 *     hardware FP32->E4M3 cast, round-to-nearest-even. The running max,
 *     its power-of-two scaling, row sums, MFMAs and repair are unchanged.
 * Any other value gives OC_ERR_INVALID_ARGUMENT and leaves the plan as it
 * was. */
typedef enum oc_weights { OC_WEIGHTS_EXPCAST = 0, OC_WEIGHTS_EXP_FP8 = 1 } oc_weights;
oc_status oc_attn_plan_set_weights(oc_attn_plan* plan, int weights);
/* K-mean smoothing for later prepare calls on this plan (host-only; default
 * off). When on, the prepare step first takes the mean key of every (b, h)
 * per channel, kbar = fp32(sum_j k_j / S) with the sum in float64, and
 * quantizes fp32(k - kbar) in place of k. q.(k - kbar) differs from q.k by a
 * constant per query row, which softmax ignores, while the K blocks lose a
 * shared bias that would otherwise widen their FP8 range. The pages name Q/K
 * smoothing as prior practice, not as part of this method (VC-Attention
 * write-up, section on why attention is the video bottleneck), so it is an
 * option. enable must be 0 or 1, else OC_ERR_INVALID_ARGUMENT. */
oc_status oc_attn_plan_set_k_smoothing(oc_attn_plan* plan, int enable);
/* V-Smooth block means for later prepare calls on this plan (host-only;
 * default off; VC-Attention write-up, section "V-Smooth", without its k-means
 * grouping of tokens). When on, each 128-token block of V loses its mean,
 * mu = bf16(fp32(sum_j v_j / n)) per channel over the block's n tokens (sum in
 * float64), and the per-head E4M3 quantization (and, with repair, the residual
 * selection) acts on fp32(v - mu). The attention on such a workspace adds the
 * means back with each key tile's row sum:
 *   O_i = (sv * sum_j P_ij dec(r_j) + sum_t l_it mu_t) / L_i.
 * oc_attn_forward_prepared follows the setting the workspace was prepared
 * with. enable must be 0 or 1, else OC_ERR_INVALID_ARGUMENT. */
oc_status oc_attn_plan_set_v_smoothing(oc_attn_plan* plan, int enable);
/* Workspace bytes the plan needs (host-only). */
oc_status oc_attn_workspace_size(const oc_attn_plan* plan, size_t* bytes);
/* Buffer offsets inside the workspace (host-only). */
oc_status oc_attn_workspace_layout(const oc_attn_plan* plan, oc_attn_ws_layout* layout);

/* Quantize q, k, v into the workspace: per-block Q/K scales and E4M3 codes,
 * per-head V scale and codes packed transposed for the matrix cores (Open VC
 * Attention product page, kernel paragraph: per-block Q/K and per-head V
 * scales; the call quantizes to FP8 itself, API paragraph). The prepare
 * kernels (two, or up to five with repair or K-mean smoothing) are launched
 * back to back on `stream`; with OC_ATTN_GRAPH=1 in the environment they run
 * instead as one captured hipGraph, replayed on later calls with the same
 * pointers (Open-VC news, "Архитектурные оптимизации": Q/K/V preparation
 * fused into one graph). On MI355X the direct launches cost less: the graph
 * launch adds about 15 us.
 * q, k, v: device, [B,S,H,128] bf16/fp16 with the plan's strides; ws: device,
 * at least oc_attn_workspace_size bytes, 256-byte aligned, overwritten;
 * stream: hipStream_t. Errors as listed at the top of this file. */
oc_status oc_attn_prepare(oc_attn_plan* plan, const void* q, const void* k, const void* v,
                          void* ws, size_t ws_bytes, void* stream);

/* Full call: oc_attn_prepare, then ExpCast attention into out (BF16,
 * contiguous [B,S,H,128], device, caller-owned). Softmax weights are E4M3
 * bytes from one FMA on the log-domain score against the bit-aligned
 * running row max, keys visited from the middle of the window (VC-Attention
 * write-up, "ExpCast-FP8"; product page, kernel paragraph); non-causal
 * attention with head dim 128 on bf16/fp16 inputs, BF16 output (product page,
 * API paragraph). Errors as listed at the top of this file. */
oc_status oc_attn_forward(oc_attn_plan* plan, const void* q, const void* k, const void* v,
                          void* out, void* ws, size_t ws_bytes, void* stream);

/* oc_attn_prepare plus the repair set for `budget` (0 <= budget <= the plan's
 * max): residual energy of every value token (sum of squares of
 * v - sv*dec(v_hat) over the channels, float64, added pairwise in channel
 * order), the top ceil(budget*S) tokens per (b, h) (ties to the lower
 * index), and their E4M3 residuals with their own per-head scale (Open-VC
 * news, "Решение: ExpCast и отказ от экспонент": repair of the worst-rounded
 * value tokens; product page, repair paragraph: prepare with a budget such
 * as 0.005). A budget outside [0, plan max] or NaN gives
 * OC_ERR_INVALID_ARGUMENT; other errors as oc_attn_prepare. */
oc_status oc_attn_prepare_v_repair(oc_attn_plan* plan, const void* q, const void* k, const void* v,
                                   double budget, void* ws, size_t ws_bytes, void* stream);

/* Full call with repair: oc_attn_prepare_v_repair, then attention whose
 * output adds the repaired residuals with the unrepaired row sums (product
 * page, repair paragraph: the repaired attention call after
 * prepare_v_repair). Arguments and errors as oc_attn_forward plus the budget
 * rule of oc_attn_prepare_v_repair. */
oc_status oc_attn_forward_v_repair(oc_attn_plan* plan, const void* q, const void* k, const void* v,
                                   double budget, void* out, void* ws, size_t ws_bytes, void* stream);

/* Capacity of the workspace inside the library used by
 * oc_attn_forward_v_repair_noalloc (per GPU): 64 MiB, enough for a plan such
 * as B=1, S=8192, H=8 with repair (oc_attn_workspace_size tells). */
#define OC_NOALLOC_WORKSPACE_BYTES (64ull << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation and result as oc_attn_forward_v_repair (budget 0: as
 * oc_attn_forward), with the workspace taken from a device array inside the
 * library instead of a caller's buffer. The call allocates nothing and
 * captures no graph: it enqueues the prepare and attention kernels directly
 * on `stream`. The array holds OC_NOALLOC_WORKSPACE_BYTES per GPU, for the
 * life of the process; a plan whose oc_attn_workspace_size exceeds that gives
 * OC_ERR_WORKSPACE_TOO_SMALL. Every call on one GPU uses that GPU's one
 * array, so calls that overlap in time on one GPU (concurrent streams, or
 * threads) race and must be serialized by the caller; consecutive calls on
 * one stream are ordered and safe. Nothing in the array needs to start at
 * zero: the prepare step writes every byte the attention reads. The first
 * call on a device, with that device current, looks up the array's address
 * there; a failing lookup gives OC_ERR_HIP. Validation as
 * oc_attn_forward_v_repair. */
oc_status oc_attn_forward_v_repair_noalloc(oc_attn_plan* plan, const void* q, const void* k, const void* v,
                                          double budget, void* out, void* stream);

/* Attention only, on a workspace this plan prepared earlier (kernel-alone
 * timing; the plan remembers its 64 most recently prepared workspaces).
 * with_repair != 0 requires the workspace to come from
 * oc_attn_prepare_v_repair; its repair set is then applied. The prepared
 * tensors are only read; the work-item counters (`sched`) are written, so
 * two calls on one workspace must not overlap. */
oc_status oc_attn_forward_prepared(oc_attn_plan* plan, void* ws, size_t ws_bytes, void* out,
                                   int with_repair, void* stream);

/* Parity aid: run the attention kernel on the prepared workspace for the
 * one (b, h) pair, every query tile of it, and record what it computed for
 * the listed query rows. out receives the normal BF16 output of that (b, h)
 * (the same bits the attention calls write there); other (b, h) pairs of out
 * are left alone.
 *   rows      device i32 [n_rows], ascending and distinct query rows
 *             (1 <= n_rows <= S; entries outside [0, S) are never matched,
 *             and an unsorted list leaves some rows unrecorded)
 *   with_repair  != 0: the workspace must come from oc_attn_prepare_v_repair,
 *             and its repair pass runs (else OC_ERR_NOT_PREPARED)
 * Each of the following device buffers may be NULL (not recorded); slot i
 * holds the row rows[i]:
 *   codes     u8  [n_rows][S]       the ExpCast byte of every key
 *   m_used    i32 [n_rows][n_ktiles] the running row max each key tile's
 *                                   bytes were written against, by tile
 *   scores    f32 [n_rows][S]       the raw FP8 MFMA sum <q_hat_i, k_hat_j>
 *                                   (codes as E4M3 values, before any scale)
 *   rcodes    u8  [n_rows][n_sel]   with_repair: the byte of every selected
 *                                   token in the repair pass (slot order)
 *   out_f32   f32 [n_rows][128]     the output row before BF16 rounding
 *                                   (16-byte aligned)
 * Same validation as oc_attn_forward_prepared, plus b, h and n_rows ranges;
 * misaligned buffers give OC_ERR_INVALID_ARGUMENT. */
oc_status oc_attn_debug_pcodes(oc_attn_plan* plan, const void* ws, size_t ws_bytes, int32_t b, int32_t h,
                               const int32_t* rows, int32_t n_rows, int32_t with_repair, uint8_t* codes,
                               int32_t* m_used, float* scores, uint8_t* rcodes, float* out_f32, void* out,
                               void* stream);

/* Static description of a status code. */
const char* oc_attn_status_string(oc_status status);
/* hipError_t of the calling thread's last OC_ERR_HIP (0 if none). */
int oc_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OC_ATTN_H */
