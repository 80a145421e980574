"""Work-item claiming of the attention kernel on long inputs.

At 4096 or more (b, h, 256-query tile) work items the last eighth of every
XCD's range of items is claimed at run time through counters in the
workspace, and stolen across XCDs once a range is used up. Every item must
run exactly once (an output filled with NaN beforehand comes back finite),
give the bits of the fixed-grid parity-aid launch of its (b, h), match the
oracle, and leave the counters at zero for the next call on the workspace.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads
from gpu_util import _oc, compare, log

pytestmark = pytest.mark.gpu

# (label, B, S, H): 4096 items in ranges of 512; 4097 items, the last range
# 7 items short; 4104 items over three batches
CASES = [("b1_s8192_h128", 1, 8192, 128), ("b1_s4300_h241", 1, 4300, 241), ("b3_s2304_h152", 3, 2304, 152)]


def claimed_items(B, S, H):
    """(b, h, query tile) of the items claimed at run time, by XCD range"""
    nqt = math.ceil(S / 256)
    nwork = B * H * nqt
    assert nwork >= 4096
    per = math.ceil(nwork / 8)
    s0 = per - per // 8
    out = []
    for x in range(8):
        items = range(x * per + s0, min(x * per + per, nwork))
        out.append([(w // (H * nqt), (w // nqt) % H, w % nqt) for w in items])
    return out


def counters(prep):
    torch.cuda.synchronize()
    return prep.tensor("sched", torch.int32, 16).cpu().numpy()


def run_twice(oc, prep, **kw):
    """two calls on one workspace, each into an output filled with NaN"""
    outs = []
    for _ in range(2):
        out = torch.full(prep.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        oc.attention_prepared(prep, out=out, **kw)
        assert not torch.isnan(out).any().item(), "an item was not run"
        assert not counters(prep).any(), counters(prep)
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    return outs[0]


def same_as_fixed_grid(oc, prep, out, pairs, **kw):
    for b, h in pairs:
        d = oc.debug_pcodes(prep, b, h, rows=[0], codes=False, m_used=False, **kw)
        assert torch.equal(d.out[b, :, h], out[b, :, h]), (b, h)


@pytest.mark.parametrize("label,B,S,H", CASES, ids=[c[0] for c in CASES])
def test_claimed_items_run_once_and_match(label, B, S, H):
    oc = _oc()
    log(f"[schedule] {label}")
    q, k, v = workloads.random_qkv(B, S, H, seed=B * 1000 + H, device="cuda", scale=1.5)
    prep = oc.prepare(q, k, v)
    assert not counters(prep).any()
    out = run_twice(oc, prep)
    ranges = claimed_items(B, S, H)
    first, last = ranges[0][0], ranges[7][-1]
    pairs = sorted({(0, 0), first[:2], last[:2], ranges[3][len(ranges[3]) // 2][:2]})
    same_as_fixed_grid(oc, prep, out, pairs)
    # oracle rows inside claimed query tiles of the first and last claimed (b, h)
    for b, h, qt in (first, last):
        rows = sorted({min(qt * 256 + r, S - 1) for r in (0, 77, 255)})
        compare(q, k, v, out, [(b, h)], rows, prep=prep, label=f"{label} claimed ({b},{h}) tile {qt}")
    # the full call (prepare, then attention) on the binding's own workspace
    assert torch.equal(oc.attention(q, k, v), out)


def test_counters_zeroed_by_prepare():
    """Counters left non-zero (as after a launch that never ended) are reset
    by the next prepare on the workspace."""
    oc = _oc()
    B, S, H = CASES[0][1:]
    q, k, v = workloads.random_qkv(B, S, H, seed=5, device="cuda")
    prep = oc.prepare(q, k, v)
    ref = run_twice(oc, prep)
    prep.tensor("sched", torch.int32, 16).fill_(1 << 20)
    assert counters(prep).all()
    st = torch.cuda.current_stream().cuda_stream
    lib, ws = oc._lib, prep.ws
    assert lib.oc_attn_prepare(prep.plan.handle, oc._ptr(q), oc._ptr(k), oc._ptr(v), oc._ptr(ws), ws.numel(), st) == 0
    assert not counters(prep).any()
    assert torch.equal(run_twice(oc, prep), ref)


@pytest.mark.parametrize("variant", ["repair", "v_smooth", "exp_fp8"])
def test_claimed_items_in_every_kernel_variant(variant):
    oc = _oc()
    label, B, S, H = CASES[1]
    log(f"[schedule] {label} {variant}")
    q, k, v = workloads.random_qkv(B, S, H, seed=11, device="cuda", scale=1.5)
    kw, okw = {}, {}
    if variant == "repair":
        prep = oc.prepare_v_repair(q, k, v, 0.01)
        kw = okw = {"with_repair": True}
    elif variant == "v_smooth":
        prep = oc.prepare(q, k, v, v_smooth=True)
    else:
        prep = oc.prepare(q, k, v)
        kw = okw = {"weights": "exp_fp8"}
    out = run_twice(oc, prep, **okw)
    ranges = claimed_items(B, S, H)
    pairs = sorted({ranges[0][0][:2], ranges[7][-1][:2], (0, H - 1)})
    same_as_fixed_grid(oc, prep, out, pairs, **kw)
    b, h, qt = ranges[7][-1]
    rows = sorted({min(qt * 256 + r, S - 1) for r in (0, 255)})
    ckw = {"budget": 0.01} if variant == "repair" else {"v_smooth": True} if variant == "v_smooth" else \
        {"weights": "exp_cast"}
    compare(q, k, v, out, [(b, h)], rows, prep=prep, label=f"{label} {variant} ({b},{h})", **ckw)
    assert np.isfinite(out[b, :, h].float().cpu().numpy()).all()


def test_claiming_kernel_replays_in_a_graph():
    """The attention call captured in a graph, on a shape whose items are
    partly claimed at run time: the counters reset themselves at the end of
    each launch, so every replay, with eager work between them, gives the
    bits of the eager call and leaves the counters at zero."""
    oc = _oc()
    label, B, S, H = CASES[0]
    q, k, v = workloads.random_qkv(B, S, H, seed=23, device="cuda")
    prep = oc.prepare(q, k, v)
    ref = run_twice(oc, prep)                       # eager calls (also configure the kernel before capture)
    out = torch.full(prep.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        oc.attention_prepared(prep, out=out)        # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            oc.attention_prepared(prep, out=out)
    torch.cuda.synchronize()
    assert not counters(prep).any()
    for i in range(3):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        assert not counters(prep).any(), (i, counters(prep))
        del junk
