"""Boundary tests that need no GPU: the library loads, exports every entry
point the header declares, sizes workspaces, and rejects bad arguments
before any HIP call (so every error path is reachable on a CPU-only host)."""
import ctypes
import math
import os
import re

import pytest

import bit_fp8_attention_block_amd as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oc_attn.h")
lib = oc._lib


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oc_attn_\w+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(oc.EXPORTS)


def make_desc(B=1, S=1000, H=4, D=128, dtype=oc.OC_BF16, strides=None, scale=0.0):
    strides = strides or (S * H * 128, H * 128, 128)
    return oc.Desc(B, S, H, D, dtype, strides[0], strides[1], strides[2], scale)


def create(desc, budget=0.0):
    p = ctypes.c_void_p()
    st = lib.oc_attn_plan_create(ctypes.byref(desc), ctypes.c_double(budget), ctypes.byref(p))
    return st, p


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), oc.OC_ERR_UNSUPPORTED),
    (dict(dtype=7), oc.OC_ERR_UNSUPPORTED),
    (dict(B=0), oc.OC_ERR_INVALID_ARGUMENT),
    (dict(S=0), oc.OC_ERR_INVALID_ARGUMENT),
    (dict(H=-1), oc.OC_ERR_INVALID_ARGUMENT),
    (dict(strides=(4000 * 128, 4 * 128, 100)), oc.OC_ERR_INVALID_ARGUMENT),
    (dict(strides=(4000 * 128, -512, 128)), oc.OC_ERR_INVALID_ARGUMENT),
    (dict(scale=math.nan), oc.OC_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), oc.OC_ERR_INVALID_ARGUMENT),
])
def test_plan_create_rejects(kw, status):
    st, p = create(make_desc(**kw))
    assert st == status and not p.value


def test_plan_create_rejects_grids_past_the_launch_limit():
    """B*H*ceil(S/256) attention workgroups must fit the 32-bit grid index."""
    st, p = create(make_desc(B=1, S=2**30, H=64))
    assert st == oc.OC_ERR_UNSUPPORTED and not p.value
    st, p = create(make_desc(B=1, S=2**30 - 256 * 16, H=16))
    assert st == oc.OC_OK and p.value
    lib.oc_attn_plan_destroy(p)


@pytest.mark.parametrize("budget", [-0.1, 1.01, math.nan])
def test_plan_create_rejects_budget(budget):
    st, p = create(make_desc(), budget)
    assert st == oc.OC_ERR_INVALID_ARGUMENT


def test_workspace_size_and_layout():
    B, S, H = 2, 73397, 3
    st, p = create(make_desc(B=B, S=S, H=H), 0.02)
    assert st == oc.OC_OK
    n = ctypes.c_size_t()
    assert lib.oc_attn_workspace_size(p, ctypes.byref(n)) == oc.OC_OK
    L = oc.WsLayout()
    assert lib.oc_attn_workspace_layout(p, ctypes.byref(L)) == oc.OC_OK
    nT, nQT = math.ceil(S / 128), math.ceil(S / 256)
    assert (L.n_ktiles, L.n_qtiles, L.s_pad_q) == (nT, nQT, nQT * 256)
    assert L.n_sel_max == 1468 and L.n_sel_tiles_max == 12
    offs = [L.qhat, L.kpack, L.vpack, L.sq, L.sk, L.vamax, L.sv, L.energy, L.sel, L.kselpack, L.rpack, L.sksel, L.sr]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert L.kpack - L.qhat >= B * H * nQT * 256 * 128
    assert L.vpack - L.kpack >= B * H * nT * 16384
    assert L.total_bytes == n.value >= L.sr + B * H * 8
    # the attention kernel's 16 work-item counters sit last, past the V-Smooth means
    assert L.sched % 256 == 0 and L.sched >= L.vmu + B * H * nT * 128 * 2 and L.total_bytes >= L.sched + 64
    lib.oc_attn_plan_destroy(p)
    st, p = create(make_desc(B=B, S=S, H=H), 0.0)
    L0 = oc.WsLayout()
    lib.oc_attn_workspace_layout(p, ctypes.byref(L0))
    assert L0.n_sel_max == 0 and L0.total_bytes < L.total_bytes
    lib.oc_attn_plan_destroy(p)


FAKE = 1 << 40          # never dereferenced: every call below fails validation first


def vp(x):
    return ctypes.c_void_p(x)


def test_forward_argument_errors_before_any_hip_call():
    st, p = create(make_desc(S=1000, H=4), 0.01)
    assert st == oc.OC_OK
    n = ctypes.c_size_t()
    lib.oc_attn_workspace_size(p, ctypes.byref(n))
    ws_bytes = n.value
    q, k, v = FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    ws, out = FAKE + (4 << 30), FAKE + (8 << 30)
    fwd = lib.oc_attn_forward
    assert fwd(p, None, vp(k), vp(v), vp(out), vp(ws), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    assert fwd(p, vp(q + 8), vp(k), vp(v), vp(out), vp(ws), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    assert fwd(p, vp(q), vp(k), vp(v), vp(out), vp(ws + 16), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    assert fwd(p, vp(q), vp(k), vp(v), vp(out), vp(ws), ws_bytes - 1, None) == oc.OC_ERR_WORKSPACE_TOO_SMALL
    # out overlapping an input or the workspace
    assert fwd(p, vp(q), vp(k), vp(v), vp(k + 256), vp(ws), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    assert fwd(p, vp(q), vp(k), vp(v), vp(ws + 1024), vp(ws), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    # workspace overlapping an input
    assert fwd(p, vp(q), vp(k), vp(v), vp(out), vp(q), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    assert fwd(None, vp(q), vp(k), vp(v), vp(out), vp(ws), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    rep = lib.oc_attn_forward_v_repair
    for b in (-0.5, 1.5, math.nan, 0.02):    # 0.02 exceeds the plan's 0.01
        assert rep(p, vp(q), vp(k), vp(v), ctypes.c_double(b), vp(out), vp(ws), ws_bytes, None) == \
            oc.OC_ERR_INVALID_ARGUMENT
    prep = lib.oc_attn_prepare_v_repair
    assert prep(p, vp(q), vp(k), vp(v), ctypes.c_double(2.0), vp(ws), ws_bytes, None) == oc.OC_ERR_INVALID_ARGUMENT
    assert lib.oc_attn_prepare(p, vp(q), vp(k), vp(v), vp(ws), 100, None) == oc.OC_ERR_WORKSPACE_TOO_SMALL
    # attention on a workspace this plan never prepared
    assert lib.oc_attn_forward_prepared(p, vp(ws), ws_bytes, vp(out), 0, None) == oc.OC_ERR_NOT_PREPARED
    assert lib.oc_attn_forward_prepared(p, vp(ws), ws_bytes, vp(out), 1, None) == oc.OC_ERR_NOT_PREPARED
    assert lib.oc_attn_forward_prepared(p, vp(ws), 10, vp(out), 0, None) == oc.OC_ERR_WORKSPACE_TOO_SMALL
    rows, codes, m = FAKE + (15 << 30), FAKE + (16 << 30), FAKE + (20 << 30)
    dbg = lib.oc_attn_debug_pcodes

    def dump(b=0, h=0, rws=rows, n=10, rep=0, cd=codes, f32=None, o=out, w=ws, nbytes=ws_bytes):
        return dbg(p, vp(w), nbytes, b, h, vp(rws), n, rep, vp(cd), vp(m), None, None, vp(f32), vp(o), None)
    assert dump() == oc.OC_ERR_NOT_PREPARED
    assert dump(rep=1) == oc.OC_ERR_NOT_PREPARED
    assert dump(h=9) == oc.OC_ERR_INVALID_ARGUMENT
    assert dump(b=-1) == oc.OC_ERR_INVALID_ARGUMENT
    assert dump(n=0) == oc.OC_ERR_INVALID_ARGUMENT
    assert dump(n=1001) == oc.OC_ERR_INVALID_ARGUMENT          # more rows than S
    assert dump(rws=None) == oc.OC_ERR_INVALID_ARGUMENT
    assert dump(rws=rows + 2) == oc.OC_ERR_INVALID_ARGUMENT      # misaligned row list
    assert dump(f32=FAKE + (24 << 30) + 4) == oc.OC_ERR_INVALID_ARGUMENT
    assert dump(o=None) == oc.OC_ERR_INVALID_ARGUMENT
    assert dump(o=ws) == oc.OC_ERR_INVALID_ARGUMENT             # output overlapping the workspace
    assert dump(nbytes=100) == oc.OC_ERR_WORKSPACE_TOO_SMALL
    lib.oc_attn_plan_destroy(p)
    lib.oc_attn_plan_destroy(None)


def test_status_strings():
    for s in range(6):
        assert lib.oc_attn_status_string(s)
    assert lib.oc_attn_last_hip_error() == 0


def test_set_weights_accepts_only_the_two_paths():
    st, p = create(make_desc())
    assert st == oc.OC_OK
    try:
        assert lib.oc_attn_plan_set_weights(p, 0) == oc.OC_OK
        assert lib.oc_attn_plan_set_weights(p, 1) == oc.OC_OK
        for bad in (-1, 2, 99):
            assert lib.oc_attn_plan_set_weights(p, bad) == oc.OC_ERR_INVALID_ARGUMENT
        assert lib.oc_attn_plan_set_weights(None, 0) == oc.OC_ERR_INVALID_ARGUMENT
    finally:
        lib.oc_attn_plan_destroy(p)
    assert oc.WEIGHTS == {"expcast": 0, "exp_fp8": 1}


def test_set_k_smoothing_accepts_0_and_1():
    st, p = create(make_desc())
    assert st == oc.OC_OK
    try:
        assert lib.oc_attn_plan_set_k_smoothing(p, 1) == oc.OC_OK
        assert lib.oc_attn_plan_set_k_smoothing(p, 0) == oc.OC_OK
        for bad in (-1, 2):
            assert lib.oc_attn_plan_set_k_smoothing(p, bad) == oc.OC_ERR_INVALID_ARGUMENT
        assert lib.oc_attn_plan_set_k_smoothing(None, 1) == oc.OC_ERR_INVALID_ARGUMENT
    finally:
        lib.oc_attn_plan_destroy(p)


def test_k_smoothing_buffers_in_layout():
    d = make_desc(B=2, S=1000, H=3)
    st, p = create(d)
    assert st == oc.OC_OK
    try:
        L = oc.WsLayout()
        assert lib.oc_attn_workspace_layout(p, ctypes.byref(L)) == oc.OC_OK
        nT = math.ceil(1000 / 128)
        assert L.kmean % 256 == 0 and L.kpart % 256 == 0
        assert L.kpart >= L.kmean + 2 * 3 * 128 * 4
        assert L.total_bytes >= L.kpart + 2 * 3 * nT * 128 * 8
    finally:
        lib.oc_attn_plan_destroy(p)


def test_set_v_smoothing_accepts_0_and_1():
    st, p = create(make_desc())
    assert st == oc.OC_OK
    try:
        assert lib.oc_attn_plan_set_v_smoothing(p, 1) == oc.OC_OK
        assert lib.oc_attn_plan_set_v_smoothing(p, 0) == oc.OC_OK
        for bad in (-1, 2):
            assert lib.oc_attn_plan_set_v_smoothing(p, bad) == oc.OC_ERR_INVALID_ARGUMENT
        assert lib.oc_attn_plan_set_v_smoothing(None, 0) == oc.OC_ERR_INVALID_ARGUMENT
        L = oc.WsLayout()
        assert lib.oc_attn_workspace_layout(p, ctypes.byref(L)) == oc.OC_OK
        nT = math.ceil(1000 / 128)
        assert L.total_bytes >= L.vmu + 4 * nT * 128 * 2
    finally:
        lib.oc_attn_plan_destroy(p)


def test_noalloc_entry_rejects_before_any_hip_call():
    """The allocation-free call checks the plan's workspace size against the
    library's array and the budget before it touches the GPU."""
    big = make_desc(B=1, S=73397, H=56)
    st, p = create(big)
    assert st == oc.OC_OK
    try:
        n = ctypes.c_size_t()
        lib.oc_attn_workspace_size(p, ctypes.byref(n))
        assert n.value > oc.NOALLOC_WORKSPACE_BYTES
        assert lib.oc_attn_forward_v_repair_noalloc(p, vp(FAKE), vp(FAKE + (1 << 33)), vp(FAKE + (1 << 34)),
                                                    ctypes.c_double(0.0), vp(FAKE + (1 << 35)), None) == \
            oc.OC_ERR_WORKSPACE_TOO_SMALL
    finally:
        lib.oc_attn_plan_destroy(p)
    st, p = create(make_desc(S=1000, H=2), 0.01)
    try:
        for b in (-0.1, 0.5, math.nan):          # 0.5 exceeds the plan's 0.01
            assert lib.oc_attn_forward_v_repair_noalloc(p, vp(FAKE), vp(FAKE), vp(FAKE), ctypes.c_double(b),
                                                        vp(FAKE), None) == oc.OC_ERR_INVALID_ARGUMENT
        assert lib.oc_attn_forward_v_repair_noalloc(None, vp(FAKE), vp(FAKE), vp(FAKE), ctypes.c_double(0.0),
                                                    vp(FAKE), None) == oc.OC_ERR_INVALID_ARGUMENT
    finally:
        lib.oc_attn_plan_destroy(p)


_LOG_CHILD = r"""
import ctypes, sys
import bit_fp8_attention_block_amd as oc
lib = oc._lib
d = oc.Desc(1, 1000, 4, 128, oc.OC_BF16, 1000 * 4 * 128, 4 * 128, 128, 0.0)
p = ctypes.c_void_p()
assert lib.oc_attn_plan_create(ctypes.byref(d), ctypes.c_double(0.01), ctypes.byref(p)) == oc.OC_OK
n = ctypes.c_size_t()
assert lib.oc_attn_workspace_size(p, ctypes.byref(n)) == oc.OC_OK
assert lib.oc_attn_plan_set_weights(p, 9) == oc.OC_ERR_INVALID_ARGUMENT
assert lib.oc_attn_forward_v_repair(p, None, None, None, ctypes.c_double(0.5), None, None, n.value,
                                    None) == oc.OC_ERR_INVALID_ARGUMENT
bad = oc.Desc(1, 1000, 4, 64, oc.OC_BF16, 1000 * 4 * 128, 4 * 128, 128, 0.0)
q = ctypes.c_void_p()
assert lib.oc_attn_plan_create(ctypes.byref(bad), ctypes.c_double(0.0), ctypes.byref(q)) == oc.OC_ERR_UNSUPPORTED
lib.oc_attn_plan_destroy(p)
print("child done")
"""


@pytest.mark.parametrize("on", [True, False])
def test_call_log_on_stderr_only_when_asked(on):
    """With OC_ATTN_LOG=1 every C-ABI call writes one line to stderr (entry
    point, shape, options, budget, status); without it, nothing."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("OC_ATTN_LOG", None)
    if on:
        env["OC_ATTN_LOG"] = "1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", _LOG_CHILD], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "child done" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("[oc_attn]")]
    if not on:
        assert lines == []
        return
    assert len(lines) == 5, lines
    assert lines[0] == "[oc_attn] oc_attn_plan_create B=1 S=1000 H=4 D=128 bf16 weights=expcast v_smooth=0 " \
                       "k_smooth=0 budget=0.01 -> ok"
    assert lines[1].startswith("[oc_attn] oc_attn_workspace_size B=1 S=1000") and lines[1].endswith("-> ok")
    assert lines[2].startswith("[oc_attn] oc_attn_plan_set_weights") and lines[2].endswith("-> invalid argument")
    assert "budget=0.5" in lines[3] and lines[3].endswith("-> invalid argument")
    assert lines[4] == "[oc_attn] oc_attn_plan_create B=1 S=1000 H=4 D=64 bf16 budget=0 -> " \
                       "unsupported (D must be 128; dtype bf16 or fp16)"
