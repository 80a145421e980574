"""The allocation-free entry point (oc_attn_forward_v_repair_noalloc),
called through the C ABI: its output equals oc_attn_forward_v_repair's on a
caller-owned workspace bit for bit, on two calls in a row where the second
has a smaller input (the library's array keeps the first call's contents),
with and without repair."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu


def _ref(oc, plan, q, k, v, budget):
    ws = torch.empty(plan.workspace_bytes + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:][:plan.workspace_bytes]
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert oc._lib.oc_attn_forward_v_repair(plan.handle, oc._ptr(q), oc._ptr(k), oc._ptr(v), ctypes.c_double(budget),
                                            oc._ptr(out), oc._ptr(ws), ws.numel(), st) == oc.OC_OK
    return out


def _noalloc(oc, plan, q, k, v, budget):
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert oc._lib.oc_attn_forward_v_repair_noalloc(plan.handle, oc._ptr(q), oc._ptr(k), oc._ptr(v),
                                                    ctypes.c_double(budget), oc._ptr(out), st) == oc.OC_OK
    return out


@pytest.mark.parametrize("budget", [0.01, 0.0])
def test_noalloc_equals_workspace_call_on_two_calls(budget):
    import bit_fp8_attention_block_amd as oc
    for name, S, H in (("s8192_h8", 8192, 8), ("b2_s70000_h40_fp16", 1000, 3)):
        log(f"[no-alloc] {name} S={S} H={H} budget={budget}")
        q, k, v = workloads.make_inputs(name, device="cuda", S=S, H=H)
        plan = oc.Plan(*q.shape[:3], q.dtype, max_budget=budget)
        assert plan.workspace_bytes <= oc.NOALLOC_WORKSPACE_BYTES
        got = _noalloc(oc, plan, q, k, v, budget)
        want = _ref(oc, plan, q, k, v, budget)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, want), name


def test_noalloc_rejects_a_plan_past_its_capacity():
    import bit_fp8_attention_block_amd as oc
    plan = oc.Plan(1, 32768, 14, torch.bfloat16)
    assert plan.workspace_bytes > oc.NOALLOC_WORKSPACE_BYTES
    q = torch.zeros(1, 32768, 14, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert oc._lib.oc_attn_forward_v_repair_noalloc(plan.handle, oc._ptr(q), oc._ptr(q), oc._ptr(q), ctypes.c_double(0),
                                                    oc._ptr(out), st) == oc.OC_ERR_WORKSPACE_TOO_SMALL


def test_noalloc_binding_matches_attention():
    import bit_fp8_attention_block_amd as oc
    q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    a = oc.attention_noalloc(q, k, v)
    b = oc.attention(q, k, v)
    c = oc.attention_noalloc(q, k, v, budget=0.005)
    d = oc.attention_v_repair(q, k, v, 0.005)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)
    assert np.isfinite(a.float().cpu().numpy()).all()
