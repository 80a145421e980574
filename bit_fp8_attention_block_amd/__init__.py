"""ExpCast FP8 forward attention for AMD Instinct MI355X (gfx950).

Thin Python binding over liboc_attn.so (C ABI in include/oc_attn.h).
PyTorch is used only to hold device memory and name the stream. Every
step of the computation runs in the library's HIP kernels, and there is no
fallback path: if the library is missing, importing the binding raises.

    out = attention(q, k, v)                     # full call: prepare + attention
    prep = prepare_v_repair(q, k, v, 0.005)      # quantize + pick repair tokens
    out = attention_v_repair(q, k, v, 0.005)     # full call with V-residual repair
    out = attention_prepared(prep, with_repair=True)   # attention on a prepared workspace
    out = attention_prepared(prep, weights="exp_fp8")  # comparison path: exp + FP8 cast
    out = attention(q, k, v, k_smooth=True)      # mean key removed before K is quantized
    out = attention(q, k, v, v_smooth=True)      # V as residuals from its 128-token block means

q, k, v: CUDA (HIP) tensors [B,S,H,128] or [S,H,128] in bf16 or fp16, with a
contiguous channel dimension and 16-byte aligned rows. The output is bf16
[B,S,H,128] (or [S,H,128]).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; OC_ATTN_LIB names another build of the same library
# (the sanitizer build the boundary tests run against)
LIB_PATH = os.environ.get("OC_ATTN_LIB") or os.path.join(_HERE, "liboc_attn.so")

OC_OK, OC_ERR_INVALID_ARGUMENT, OC_ERR_UNSUPPORTED, OC_ERR_WORKSPACE_TOO_SMALL, OC_ERR_NOT_PREPARED, OC_ERR_HIP = range(6)
OC_BF16, OC_FP16 = 0, 1
# softmax-weight paths (oc_weights): ExpCast bytes, or exponential + FP32->E4M3 cast
WEIGHTS = {"expcast": 0, "exp_fp8": 1}


class OcAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("stride_b", ctypes.c_int64), ("stride_s", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("softmax_scale", ctypes.c_float)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("qhat", "kpack", "vpack", "sq", "sk", "vamax", "sv", "energy", "sel",
                                               "kselpack", "rpack", "sksel", "sr", "kmean", "kpart", "vmu",
                                               "sched", "total_bytes")] + \
               [(n, ctypes.c_int32) for n in ("n_ktiles", "n_qtiles", "s_pad_q", "n_sel_max", "n_sel_tiles_max")]


EXPORTS = ("oc_attn_plan_create", "oc_attn_plan_destroy", "oc_attn_workspace_size", "oc_attn_workspace_layout",
           "oc_attn_prepare", "oc_attn_forward", "oc_attn_prepare_v_repair", "oc_attn_forward_v_repair",
           "oc_attn_forward_prepared", "oc_attn_debug_pcodes", "oc_attn_status_string", "oc_attn_last_hip_error",
           "oc_attn_plan_set_weights", "oc_attn_plan_set_k_smoothing", "oc_attn_plan_set_v_smoothing",
           "oc_attn_forward_v_repair_noalloc")
# workspace capacity of oc_attn_forward_v_repair_noalloc (per GPU)
NOALLOC_WORKSPACE_BYTES = 64 << 20


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python bit_fp8_attention_block_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, VP, SZ, I32, I64, D = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    st = ctypes.c_int
    lib.oc_attn_plan_create.argtypes = [ctypes.POINTER(Desc), D, ctypes.POINTER(P)]
    lib.oc_attn_plan_destroy.argtypes = [P]
    lib.oc_attn_plan_destroy.restype = None
    lib.oc_attn_plan_set_weights.argtypes = [P, ctypes.c_int]
    lib.oc_attn_plan_set_k_smoothing.argtypes = [P, ctypes.c_int]
    lib.oc_attn_plan_set_v_smoothing.argtypes = [P, ctypes.c_int]
    lib.oc_attn_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.oc_attn_workspace_layout.argtypes = [P, ctypes.POINTER(WsLayout)]
    lib.oc_attn_prepare.argtypes = [P, VP, VP, VP, VP, SZ, VP]
    lib.oc_attn_forward.argtypes = [P, VP, VP, VP, VP, VP, SZ, VP]
    lib.oc_attn_prepare_v_repair.argtypes = [P, VP, VP, VP, D, VP, SZ, VP]
    lib.oc_attn_forward_v_repair.argtypes = [P, VP, VP, VP, D, VP, VP, SZ, VP]
    lib.oc_attn_forward_prepared.argtypes = [P, VP, SZ, VP, ctypes.c_int, VP]
    lib.oc_attn_forward_v_repair_noalloc.argtypes = [P, VP, VP, VP, D, VP, VP]
    lib.oc_attn_debug_pcodes.argtypes = [P, VP, SZ, I32, I32, VP, I32, I32, VP, VP, VP, VP, VP, VP, VP]
    lib.oc_attn_status_string.argtypes = [st]
    lib.oc_attn_status_string.restype = ctypes.c_char_p
    lib.oc_attn_last_hip_error.argtypes = []
    for name in ("oc_attn_plan_create", "oc_attn_plan_set_weights", "oc_attn_plan_set_k_smoothing",
                 "oc_attn_plan_set_v_smoothing",
                 "oc_attn_workspace_size", "oc_attn_workspace_layout", "oc_attn_prepare",
                 "oc_attn_forward", "oc_attn_prepare_v_repair", "oc_attn_forward_v_repair",
                 "oc_attn_forward_prepared", "oc_attn_debug_pcodes", "oc_attn_forward_v_repair_noalloc"):
        getattr(lib, name).restype = st
    del I64
    return lib


_lib = load_library()


def _check(status, what):
    if status != OC_OK:
        msg = _lib.oc_attn_status_string(status).decode()
        if status == OC_ERR_HIP:
            msg += f" (hipError_t {_lib.oc_attn_last_hip_error()})"
        raise OcAttnError(status, f"{what}: {msg}")


def _set_weights(plan, weights):
    if weights not in WEIGHTS:
        raise OcAttnError(OC_ERR_INVALID_ARGUMENT, f"weights must be one of {sorted(WEIGHTS)}")
    _check(_lib.oc_attn_plan_set_weights(plan.handle, WEIGHTS[weights]), "oc_attn_plan_set_weights")


def _set_smoothing(plan, k_smooth, v_smooth):
    _check(_lib.oc_attn_plan_set_k_smoothing(plan.handle, int(bool(k_smooth))), "oc_attn_plan_set_k_smoothing")
    _check(_lib.oc_attn_plan_set_v_smoothing(plan.handle, int(bool(v_smooth))), "oc_attn_plan_set_v_smoothing")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Plan:
    """One problem shape (and repair budget capacity) of the library."""

    def __init__(self, B, S, H, dtype=torch.bfloat16, strides=None, softmax_scale=0.0, max_budget=0.0):
        if strides is None:
            strides = (S * H * 128, H * 128, 128)
        dt = {torch.bfloat16: OC_BF16, torch.float16: OC_FP16}.get(dtype, 99)
        self.desc = Desc(B, S, H, 128, dt, strides[0], strides[1], strides[2], float(softmax_scale or 0.0))
        self.max_budget = float(max_budget)
        self._p = ctypes.c_void_p()
        self._lib = _lib   # the library that owns the plan also destroys it
        _check(_lib.oc_attn_plan_create(ctypes.byref(self.desc), ctypes.c_double(self.max_budget),
                                        ctypes.byref(self._p)), "oc_attn_plan_create")
        n = ctypes.c_size_t()
        _check(_lib.oc_attn_workspace_size(self._p, ctypes.byref(n)), "oc_attn_workspace_size")
        self.workspace_bytes = n.value
        self.layout = WsLayout()
        _check(_lib.oc_attn_workspace_layout(self._p, ctypes.byref(self.layout)), "oc_attn_workspace_layout")

    def __del__(self):
        p, lib = getattr(self, "_p", None), getattr(self, "_lib", None)
        if p is not None and p.value and lib is not None:
            lib.oc_attn_plan_destroy(p)
            self._p = None

    @property
    def handle(self):
        return self._p


def _canon(q, k, v):
    if q.dim() == 3:
        q, k, v = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
        squeeze = True
    else:
        squeeze = False
    if q.dim() != 4 or q.shape[-1] != 128:
        raise OcAttnError(OC_ERR_UNSUPPORTED, "inputs must be [B,S,H,128] or [S,H,128]")
    if not (q.shape == k.shape == v.shape and q.stride() == k.stride() == v.stride()):
        raise OcAttnError(OC_ERR_INVALID_ARGUMENT, "q, k, v must share shape and strides")
    if not (q.dtype == k.dtype == v.dtype) or not q.is_cuda:
        raise OcAttnError(OC_ERR_INVALID_ARGUMENT, "q, k, v must be GPU tensors of one dtype")
    if q.stride(-1) != 1:
        raise OcAttnError(OC_ERR_INVALID_ARGUMENT, "channel dimension must be contiguous")
    return q, k, v, squeeze


class Prepared:
    """A workspace filled by prepare / prepare_v_repair, with its plan.
    budget is None for a plain prepare."""

    def __init__(self, plan, ws, shape, device, budget, softmax_scale):
        self.plan, self.ws, self.shape, self.device = plan, ws, shape, device
        self.budget, self.softmax_scale = budget, softmax_scale

    @property
    def n_sel(self):
        """selected tokens per (b, h): ceil(budget*S), as the library counts them"""
        if not self.budget:
            return 0
        S = self.shape[1]
        return max(0, min(S, math.ceil(self.budget * S - 1e-9)))

    def tensor(self, name, dtype, count):
        off = getattr(self.plan.layout, name)
        nbytes = count * torch.empty(0, dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype)


_PLANS: dict = {}


def get_plan(q, softmax_scale=None, max_budget=0.0):
    B, S, H, _ = q.shape
    key = (B, S, H, q.dtype, tuple(q.stride()[:3]), float(softmax_scale or 0.0), float(max_budget), q.device)
    pl = _PLANS.get(key)
    if pl is None:
        pl = Plan(B, S, H, q.dtype, q.stride()[:3], softmax_scale or 0.0, max_budget)
        if len(_PLANS) > 16:
            _PLANS.clear()
        _PLANS[key] = pl
    return pl


def _workspace(plan, device):
    """The plan's workspace for the current stream of `device`: calls of one
    shape on different streams get different workspaces, so they may run
    concurrently (calls on one stream are ordered by the stream)."""
    stream = torch.cuda.current_stream(device).cuda_stream
    cache = plan.__dict__.setdefault("_ws", {})
    ws = cache.get((device, stream))
    if ws is None:
        ws = torch.empty(plan.workspace_bytes + 256, dtype=torch.uint8, device=device)
        pad = (-ws.data_ptr()) % 256
        ws = ws[pad:pad + plan.workspace_bytes]
        cache[(device, stream)] = ws
    return ws


def prepare(q, k, v, budget=None, softmax_scale=None, k_smooth=False, v_smooth=False) -> Prepared:
    """Quantize q, k, v into a workspace owned by the returned object. With a
    budget (prepare_v_repair), also rank the value tokens by residual energy
    and quantize the residuals of the top ceil(budget*S) of every (b, h).
    k_smooth subtracts the mean key of every (b, h) before quantizing K;
    v_smooth quantizes V as residuals from its 128-token block means."""
    q, k, v, _ = _canon(q, k, v)
    plan = get_plan(q, softmax_scale, budget or 0.0)
    _set_smoothing(plan, k_smooth, v_smooth)
    ws = torch.empty(plan.workspace_bytes + 256, dtype=torch.uint8, device=q.device)
    pad = (-ws.data_ptr()) % 256
    ws = ws[pad:pad + plan.workspace_bytes]
    st = _stream(q.device)
    if budget is not None:
        _check(_lib.oc_attn_prepare_v_repair(plan.handle, _ptr(q), _ptr(k), _ptr(v), ctypes.c_double(budget),
                                             _ptr(ws), ws.numel(), st), "oc_attn_prepare_v_repair")
    else:
        _check(_lib.oc_attn_prepare(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(ws), ws.numel(), st),
               "oc_attn_prepare")
    return Prepared(plan, ws, tuple(q.shape), q.device, budget, softmax_scale)


def prepare_v_repair(q, k, v, budget, softmax_scale=None, k_smooth=False, v_smooth=False) -> Prepared:
    return prepare(q, k, v, budget, softmax_scale, k_smooth, v_smooth)


def attention(q, k, v, softmax_scale=None, out=None, weights="expcast", k_smooth=False, v_smooth=False):
    """Full call: FP8 quantization + ExpCast attention, BF16 output.
    weights="exp_fp8" runs the comparison path (exponential + FP8 cast);
    k_smooth subtracts the mean key before quantizing K; v_smooth quantizes V
    as residuals from its block means and adds the means back per key tile."""
    q, k, v, squeeze = _canon(q, k, v)
    plan = get_plan(q, softmax_scale, 0.0)
    _set_weights(plan, weights)
    _set_smoothing(plan, k_smooth, v_smooth)
    ws = _workspace(plan, q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check(_lib.oc_attn_forward(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws), ws.numel(),
                                _stream(q.device)), "oc_attn_forward")
    return out.squeeze(0) if squeeze else out


def attention_v_repair(q, k, v, budget, softmax_scale=None, out=None, weights="expcast", k_smooth=False,
                       v_smooth=False):
    """Full call with V-residual repair of the ceil(budget*S) worst-rounded
    value tokens of every (b, h)."""
    q, k, v, squeeze = _canon(q, k, v)
    plan = get_plan(q, softmax_scale, budget)
    _set_weights(plan, weights)
    _set_smoothing(plan, k_smooth, v_smooth)
    ws = _workspace(plan, q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check(_lib.oc_attn_forward_v_repair(plan.handle, _ptr(q), _ptr(k), _ptr(v), ctypes.c_double(budget), _ptr(out),
                                         _ptr(ws), ws.numel(), _stream(q.device)), "oc_attn_forward_v_repair")
    return out.squeeze(0) if squeeze else out


def attention_noalloc(q, k, v, budget=0.0, softmax_scale=None, out=None, weights="expcast"):
    """Full call (with repair when budget > 0) on the library's own workspace
    array instead of a torch-allocated one (oc_attn_forward_v_repair_noalloc):
    for shapes whose workspace fits NOALLOC_WORKSPACE_BYTES. Calls that
    overlap in time on one GPU race on that array."""
    q, k, v, squeeze = _canon(q, k, v)
    plan = get_plan(q, softmax_scale, budget)
    _set_weights(plan, weights)
    _set_smoothing(plan, False, False)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    with torch.cuda.device(q.device):
        _check(_lib.oc_attn_forward_v_repair_noalloc(plan.handle, _ptr(q), _ptr(k), _ptr(v), ctypes.c_double(budget),
                                                     _ptr(out), _stream(q.device)), "oc_attn_forward_v_repair_noalloc")
    return out.squeeze(0) if squeeze else out


def attention_prepared(prep: Prepared, with_repair=None, out=None, weights="expcast"):
    """Attention only, on a workspace filled by prepare / prepare_v_repair.
    The call writes the workspace's work-item counters, so calls on one
    Prepared must be ordered (one stream, or synchronized streams)."""
    _set_weights(prep.plan, weights)
    if with_repair is None:
        with_repair = prep.budget is not None
    if out is None:
        out = torch.empty(prep.shape, dtype=torch.bfloat16, device=prep.device)
    _check(_lib.oc_attn_forward_prepared(prep.plan.handle, _ptr(prep.ws), prep.ws.numel(), _ptr(out),
                                         int(bool(with_repair)), _stream(prep.device)), "oc_attn_forward_prepared")
    return out


class Dump:
    """What the attention kernel computed for the listed query rows of one
    (b, h) (oc_attn_debug_pcodes). Arrays are device tensors, row i of each
    belonging to rows[i]; fields not asked for are None.
      codes   u8  [n, S]       ExpCast bytes of the main loop
      m_used  i32 [n, nT]      running row max used for each key tile, by tile
      scores  f32 [n, S]       raw FP8 MFMA sums <q_hat, k_hat>
      rcodes  u8  [n, n_sel]   repair-pass bytes (with_repair)
      out_f32 f32 [n, 128]     output rows before BF16 rounding
      out     bf16, the full output tensor; only (b, h) is written"""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def debug_pcodes(prep: Prepared, b: int, h: int, rows=None, codes=True, m_used=True, scores=False, out_f32=False,
                 with_repair=False, weights="expcast") -> Dump:
    """Run the attention kernel's parity-aid variant on a prepared workspace
    for one (b, h) and record its bytes, running maxima, raw scores, repair
    bytes and fp32 output rows for the given query rows (default: all)."""
    _set_weights(prep.plan, weights)
    B, S, H, _ = prep.shape
    dev = prep.device
    nT = prep.plan.layout.n_ktiles
    rows_t = torch.arange(S, dtype=torch.int32, device=dev) if rows is None else \
        torch.as_tensor(rows, dtype=torch.int32).to(dev)
    n = rows_t.numel()
    n_sel = 0
    if with_repair:
        if prep.budget is None:
            raise OcAttnError(OC_ERR_NOT_PREPARED, "with_repair needs a workspace from prepare_v_repair")
        n_sel = prep.n_sel
    d = Dump(rows=rows_t,
             codes=torch.zeros((n, S), dtype=torch.uint8, device=dev) if codes else None,
             m_used=torch.full((n, nT), -(1 << 30), dtype=torch.int32, device=dev) if m_used else None,
             scores=torch.full((n, S), float("nan"), dtype=torch.float32, device=dev) if scores else None,
             rcodes=torch.zeros((n, max(n_sel, 1)), dtype=torch.uint8, device=dev) if with_repair else None,
             out_f32=torch.full((n, 128), float("nan"), dtype=torch.float32, device=dev) if out_f32 else None,
             out=torch.zeros(prep.shape, dtype=torch.bfloat16, device=dev))
    _check(_lib.oc_attn_debug_pcodes(prep.plan.handle, _ptr(prep.ws), prep.ws.numel(), b, h, _ptr(rows_t), n,
                                     int(bool(with_repair)), _ptr(d.codes), _ptr(d.m_used), _ptr(d.scores),
                                     _ptr(d.rcodes), _ptr(d.out_f32), _ptr(d.out), _stream(dev)),
           "oc_attn_debug_pcodes")
    if d.rcodes is not None:
        d.rcodes = d.rcodes[:, :n_sel]
    return d


def flops(B, S, H, D=128):
    """Attention FLOPs counted as 4*B*S^2*H*D (QK^T and PV)."""
    return 4.0 * B * S * S * H * D


__all__ = ["attention", "attention_v_repair", "attention_noalloc", "prepare", "prepare_v_repair", "attention_prepared", "debug_pcodes", "Dump",
           "Plan", "Prepared", "OcAttnError", "flops", "load_library", "EXPORTS", "LIB_PATH", "WEIGHTS"]
