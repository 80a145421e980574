"""Attention kernel vs the oracle.

* ExpCast bytes: the kernel's own bytes (debug dump) against the oracle's
  bytes for the same logits and the running row max the kernel used: at
  least 99.9% equal, never more than one code apart (the remaining
  differences come from the kernel's logits, summed by the FP8 MFMA and
  scaled in fp32, against float64 in the oracle).
* Output: relative L2 against the oracle <= 5e-3, at every workload size
  (all rows on the small ones, sampled rows, always including the ragged tail,
  on the large ones, in the launch configuration the benchmark times).
* Edge cases: one key, ragged tails, identical keys, [S,H,128] inputs,
  strided inputs, batch > 1, fp16; determinism and graph replays.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (KERNEL_WEIGHTS, TOL, _oc, check_max_trace, compare, head64, kernel_dump,  # noqa: F401
                      log, logit_error_bound, oracle_rows, out_rows, validated_codes)

pytestmark = pytest.mark.gpu

# helpers shared by the GPU parity tests (also imported from here by older call sites)
_compare = compare


def check_bytes(q, k, v, prep, b, h, rows, out=None, weights="expcast", tau=None, label=""):
    """The kernel's bytes for the given rows of (b, h) against the oracle's
    bytes for the same logits and the running max the kernel used for each
    key (validated first): at least 99.9% equal, never more than one code
    apart. The final running max is the bit-aligned row max up to a tie
    within the logit error bound. Returns the dump."""
    tau = tau or 1 / math.sqrt(128)
    S = q.shape[1]
    d = kernel_dump(prep, b, h, rows, out=out, weights=weights)
    ph = oracle.prepare_head(head64(q, b, h), head64(k, b, h), head64(v, b, h))
    x = oracle.log2_logits(ph, rows, tau)
    bound = logit_error_bound(ph, rows, tau)
    ties = check_max_trace(d.m_used, x, bound)
    Mk = d.m_used[:, np.arange(S) // 128]              # running max used for each (row, key)
    want = (oracle.expcast_codes if weights == "expcast" else oracle.exp_cast_codes)(x, Mk)
    diff = np.abs(d.codes.astype(int) - want.astype(int))
    agree = (diff == 0).mean()
    log(f"  {label} (b={b},h={h}) {len(rows)} rows: byte agreement {agree:.6f}, max diff {diff.max()}, "
        f"tie-broken rows {ties}")
    assert agree >= 0.999 and diff.max() <= 1, (agree, diff.max())
    # and every differing byte is one a logit within the error bound gives
    validated_codes(d.codes, x, Mk.astype(np.float64), bound, weights)
    Mfinal = d.m_used.max(axis=1)
    Mo = oracle.bitaligned_row_max(x)
    xmax = x.max(axis=1)
    for i in np.nonzero(Mfinal != Mo)[0]:
        gap = abs(xmax[i] - round(xmax[i]))
        log(f"  row {rows[i]}: kernel M {Mfinal[i]} oracle M {Mo[i]} (max logit {xmax[i]:.9f})")
        assert abs(int(Mfinal[i]) - int(Mo[i])) == 1 and gap <= bound[i].max()
    d.x, d.ph, d.agree = x, ph, agree
    return d


@pytest.mark.parametrize("case", ["s1024_h2", "ragged300", "s130", "biased2048"])
def test_expcast_bytes_match_oracle(case):
    oc = _oc()
    log(f"[bytes] case={case}")
    if case == "s1024_h2":
        q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    elif case == "ragged300":
        q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=300, H=2)
    elif case == "s130":
        q, k, v = workloads.random_qkv(1, 130, 1, seed=4, device="cuda", scale=2.0)
    else:
        q, k, v = workloads.make_inputs("s73397_h56", device="cuda", S=2048, H=2)
    B, S, H, _ = q.shape
    out = oc.attention(q, k, v)
    prep = oc.prepare(q, k, v)
    for b in range(B):
        for h in range(H):
            d = check_bytes(q, k, v, prep, b, h, np.arange(S), out=out, label=case)
            r = oracle.expcast_attention_online(head64(q, b, h), head64(k, b, h), head64(v, b, h), ph=d.ph,
                                                m_trace=d.m_used)
            e = oracle.rel_l2(out_rows(out, b, h, np.arange(S)), r["out"])
            assert e <= TOL, e


@pytest.mark.parametrize("name,rows_per_head,pairs", [
    ("s8192_h8", 1024, "all"),
    ("s32768_h14", 128, [(0, 0), (0, 6), (0, 13)]),
    ("s73397_h56", 96, [(0, 0), (0, 27), (0, 55)]),
    ("b2_s70000_h40_fp16", 96, [(0, 0), (1, 39)]),
])
def test_expcast_bytes_match_oracle_at_full_size(name, rows_per_head, pairs):
    """Byte parity on the full workloads, in the launch configuration the
    benchmark times: every key of sampled query rows (the ragged tail
    included), on every head of s8192_h8 and on heads across the others."""
    oc = _oc()
    w = workloads.WORKLOADS[name]
    log(f"[bytes full size] {name} B={w.B} S={w.S} H={w.H}")
    q, k, v = workloads.make_inputs(name, device="cuda")
    out = oc.attention(q, k, v)
    prep = oc.prepare(q, k, v)
    rows = np.array(workloads.sample_rows(w.S, rows_per_head, seed=w.seed))
    if pairs == "all":
        pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in pairs:
        check_bytes(q, k, v, prep, b, h, rows, out=out, label=name)


@pytest.mark.parametrize("name,rows_per_head,pairs", [
    ("s1024_h2", None, "all"),
    ("s8192_h8", 512, "all"),
    ("s32768_h14", 192, [(0, 0), (0, 7), (0, 13)]),
    ("s73397_h56", 96, [(0, 0), (0, 31), (0, 55)]),
    ("b2_s70000_h40_fp16", 96, [(0, 0), (1, 17), (1, 39)]),
])
def test_output_matches_oracle_on_workloads(name, rows_per_head, pairs):
    oc = _oc()
    w = workloads.WORKLOADS[name]
    log(f"[workload] {name} B={w.B} S={w.S} H={w.H}")
    q, k, v = workloads.make_inputs(name, device="cuda")
    out = oc.attention(q, k, v)
    prep = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    B, S, H, _ = q.shape
    rows = np.arange(S) if rows_per_head is None else np.array(workloads.sample_rows(S, rows_per_head, seed=w.seed))
    if pairs == "all":
        pairs = [(b, h) for b in range(B) for h in range(H)]
    _compare(q, k, v, out, pairs, rows, label=name, prep=prep)


@pytest.mark.parametrize("S", [1, 2, 3, 127, 129, 255, 257, 511])
def test_ragged_and_tiny_sequences(S):
    oc = _oc()
    log(f"[ragged] S={S}")
    q, k, v = workloads.random_qkv(2, S, 3, seed=S, device="cuda", scale=1.5)
    out = oc.attention(q, k, v)
    torch.cuda.synchronize()
    _compare(q, k, v, out, [(0, 0), (1, 2)], np.arange(S), label=f"S={S}")


def test_single_key_returns_dequantized_value():
    oc = _oc()
    q, k, v = workloads.random_qkv(1, 1, 2, seed=1, device="cuda")
    out = oc.attention(q, k, v)
    torch.cuda.synchronize()
    for h in range(2):
        ph = oracle.prepare_head(head64(q, 0, h), head64(k, 0, h), head64(v, 0, h))
        want = float(ph.sv) * oracle.decode(ph.vc[0])
        got = out[0, 0, h].float().cpu().numpy()
        np.testing.assert_allclose(got, want, rtol=2 ** -8, atol=1e-30)


def test_identical_keys_give_mean_value():
    oc = _oc()
    S = 700
    q, k, v = workloads.random_qkv(1, S, 1, seed=2, device="cuda")
    k[:] = k[:, :1]
    out = oc.attention(q, k, v)
    torch.cuda.synchronize()
    ph = oracle.prepare_head(head64(q, 0, 0), head64(k, 0, 0), head64(v, 0, 0))
    mean = float(ph.sv) * oracle.decode(ph.vc).mean(axis=0)
    got = out[0, :, 0].float().cpu().numpy()
    assert oracle.rel_l2(got, np.tile(mean, (S, 1))) < 4e-3


@pytest.mark.parametrize("variant", ["expcast", "exp_fp8", "repair", "vsmooth", "vsmooth_tiny_v"])
def test_running_max_rising_by_many_binades(variant):
    """The kernel keeps O and L in the frame of a reference max and re-anchors
    them (by an exact power of two) once the running max has risen more than
    64 binades past it. Here the first 16 queries of every 32 see their max
    rise by about 41 binades at each key tile they visit: those queries hold
    2 in channels 0-63 and the keys of the i-th visited tile 2.5*i there, so
    their frame is re-anchored with O and L already non-zero, while the other
    16 queries of the same waves behave normally. (The large logit is spread
    over 64 equal products: a single dominant product would instead test the
    FP8 MFMA's summation precision, which is coarser than fp32.) With V-Smooth
    the row sums waiting for the next mean-term batch are re-anchored too; its
    20 tiles put a batch boundary among the re-anchors. With values of size
    1e-20, 448/amax is about 2^73 and the row sums near the frame's limit:
    the mean term must move that factor onto the means to stay finite."""
    oc = _oc()
    S = 2560 if variant.startswith("vsmooth") else 1024
    g = torch.Generator().manual_seed(31)
    q = torch.randn(1, S, 1, 128, generator=g) * 0.5
    k = torch.randn(1, S, 1, 128, generator=g) * 0.5
    v = torch.randn(1, S, 1, 128, generator=g)
    rising = torch.as_tensor((np.arange(S) % 32) < 16)
    q[0, rising, 0, :64] = 2.0
    for i, t in enumerate(oracle.key_tile_order(S // 128)):
        k[0, 128 * t:128 * (t + 1), 0, :64] = 2.5 * i
    if variant == "vsmooth_tiny_v":
        v = v * 1e-20
    q, k, v = (x.to(torch.bfloat16).cuda() for x in (q, k, v))
    log(f"[rising max] variant={variant}")
    if variant == "repair":
        prep = oc.prepare_v_repair(q, k, v, 0.02)
        out = oc.attention_v_repair(q, k, v, 0.02)
        opts = dict(budget=0.02)
    elif variant.startswith("vsmooth"):
        prep = oc.prepare(q, k, v, v_smooth=True)
        out = oc.attention(q, k, v, v_smooth=True)
        opts = dict(v_smooth=True)
    else:
        prep = oc.prepare(q, k, v)
        out = oc.attention(q, k, v, weights=variant)
        opts = dict(weights="exp_cast" if variant == "exp_fp8" else "expcast")
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    _compare(q, k, v, out, [(0, 0)], np.arange(S), label=f"rising max ({variant})", prep=prep, **opts)


def test_three_dim_and_strided_inputs():
    oc = _oc()
    S, H = 640, 2
    qkv = torch.randn(S, 3, H, 128, device="cuda").to(torch.float16)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    out = oc.attention(q, k, v)
    torch.cuda.synchronize()
    assert out.shape == (S, H, 128) and out.dtype == torch.bfloat16
    _compare(q[None], k[None], v[None], out[None], [(0, 0), (0, 1)], np.arange(0, S, 3), label="strided 3-D")


def test_softmax_scale_argument():
    oc = _oc()
    q, k, v = workloads.random_qkv(1, 400, 1, seed=8, device="cuda")
    out = oc.attention(q, k, v, softmax_scale=0.3)
    torch.cuda.synchronize()
    r = oracle.expcast_attention_online(head64(q, 0, 0), head64(k, 0, 0), head64(v, 0, 0), tau=0.3)
    assert oracle.rel_l2(out_rows(out, 0, 0, np.arange(400)), r["out"]) <= TOL


@pytest.fixture
def prepare_graph(request, monkeypatch):
    """OC_ATTN_GRAPH for the test (read by the library on every prepare)."""
    if request.param:
        monkeypatch.setenv("OC_ATTN_GRAPH", "1")
    else:
        monkeypatch.delenv("OC_ATTN_GRAPH", raising=False)
    return request.param


@pytest.mark.parametrize("prepare_graph", [False, True], indirect=True)
def test_deterministic_and_graph_replays(prepare_graph, monkeypatch):
    """Repeated calls give the same bits, with eager work in between; with
    the prepare graph (OC_ATTN_GRAPH=1) every call after the first replays it,
    and new pointers re-capture it. The direct launches and the graph give
    the same bits."""
    oc = _oc()
    q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=4096, H=4)
    ref = oc.attention(q, k, v).clone()
    for i in range(4):
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between calls
        out = oc.attention(q, k, v)                            # same pointers: graph replay
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        del junk
    out = oc.attention(q.clone(), k, v)                        # new pointers: graph re-capture
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    prep = oc.prepare(q, k, v)
    o2 = oc.attention_prepared(prep)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref)
    rep = oc.attention_v_repair(q, k, v, 0.01).clone()
    for i in range(3):
        assert torch.equal(oc.attention_v_repair(q, k, v, 0.01), rep), i
    if prepare_graph:
        monkeypatch.delenv("OC_ATTN_GRAPH")
        assert torch.equal(oc.attention(q, k, v), ref)             # direct launches, same bits
        assert torch.equal(oc.attention_v_repair(q, k, v, 0.01), rep)


def test_traversal_orders_match_their_oracle():
    """Mid-window and ascending key-tile orders each match the single-pass
    oracle run in the same order; they differ from each other only through
    the underflow tail (the bit-aligned max makes every rescale exact)."""
    import ctypes
    import os
    oc = _oc()
    q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=3000, H=2)
    outs = []
    for order in ("0", "1"):
        os.environ["OC_ATTN_ORDER"] = order
        try:
            plan = oc.Plan(1, 3000, 2, torch.bfloat16)
        finally:
            os.environ.pop("OC_ATTN_ORDER")
        ws = torch.empty(plan.workspace_bytes + 256, dtype=torch.uint8, device="cuda")
        ws = ws[(-ws.data_ptr()) % 256:][:plan.workspace_bytes]
        out = torch.empty_like(q)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert oc._lib.oc_attn_forward(plan.handle, oc._ptr(q), oc._ptr(k), oc._ptr(v), oc._ptr(out), oc._ptr(ws),
                                       ws.numel(), st) == 0
        torch.cuda.synchronize()
        outs.append(out.float())
        _compare(q, k, v, out, [(0, 0), (0, 1)], np.arange(0, 3000, 11),
                 order="mid" if order == "0" else "ascending", label=f"order {order}")
    d = (outs[0] - outs[1]).norm() / outs[1].norm()
    log(f"  mid-window vs ascending rel-L2 {d.item():.2e}")


def test_very_negative_logits_stay_finite():
    """Rows whose log2-logits all lie near -1.6e5, far below any finite
    starting value a running max could be given: every key is the same
    vector, so each row's weights are uniform and its output is the mean of
    the dequantized values, for the kernel as for the oracle."""
    oc = _oc()
    S, H = 600, 2
    g = torch.Generator().manual_seed(41)
    w = torch.randint(0, 2, (H, 128), generator=g).float() * 2 - 1                # +-1 per channel
    flips = (torch.rand(S, H, 128, generator=g) < 0.05).float() * -2 + 1
    q = (-100.0 * w[None] * flips)[None]                                           # q.k = -1e4 * (128 - 2 flips)
    k = (100.0 * w)[None, None].expand(1, S, H, 128).contiguous()
    v = torch.randn(1, S, H, 128, generator=g)
    q, k, v = (t.to(torch.bfloat16).cuda() for t in (q, k, v))
    log("[range] very negative logits")
    out = oc.attention(q, k, v)
    prep = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    for h in range(H):
        ph = oracle.prepare_head(head64(q, 0, h), head64(k, 0, h), head64(v, 0, h))
        x = oracle.log2_logits(ph, np.arange(0, S, 37), 1 / math.sqrt(128))
        assert x.max() < -1e5
        mean = float(ph.sv) * oracle.decode(ph.vc).mean(axis=0)
        got = out_rows(out, 0, h, np.arange(S))
        e = oracle.rel_l2(got, np.tile(mean, (S, 1)))
        log(f"  h={h}: rel-L2 vs the mean value {e:.2e}")
        assert e <= TOL
    compare(q, k, v, out, [(0, 0), (0, 1)], np.arange(0, S, 5), label="very negative logits", prep=prep)


def test_repair_with_tiny_residuals_stays_finite():
    """Values exactly on the E4M3 grid of their head scale (residual 0)
    except one element of 2^-90: the selected residuals are ~2^-99 of the
    head's value scale. The repaired output must stay finite and match the
    oracle; a kernel that multiplied its accumulator by that ratio would
    overflow fp32."""
    oc = _oc()
    S, H, budget = 700, 1, 0.01
    g = torch.Generator().manual_seed(42)
    grid = torch.tensor(oracle.VALUES[:127], dtype=torch.float32)
    v = grid[torch.randint(0, 127, (1, S, H, 128), generator=g)] * (torch.randint(0, 2, (1, S, H, 128), generator=g) * 2 - 1)
    v[0, 3, 0, 0] = 448.0                  # head amax 448: scale 1, every value exact
    v[0, 250, 0, 7] = 2.0 ** -90           # rounds to code 0: the one non-zero residual
    q, k, _ = workloads.make_inputs("s8192_h8", S=S, H=H)
    q, k, v = q.cuda(), k.cuda(), v.to(torch.bfloat16).cuda()
    log("[range] tiny residuals")
    out = oc.attention_v_repair(q, k, v, budget)
    prep = oc.prepare_v_repair(q, k, v, budget)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rp = oracle.prepare_head(head64(q, 0, 0), head64(k, 0, 0), head64(v, 0, 0), budget).repair
    assert 250 in rp.sel and float(rp.sr) < 2.0 ** -90 / 400
    compare(q, k, v, out, [(0, 0)], np.arange(0, S, 3), budget=budget, label="tiny residuals", prep=prep)


@pytest.mark.parametrize("name,rows_per_head,pairs", [
    ("s32768_h14", 192, [(0, 0), (0, 7), (0, 13)]),
    ("s73397_h56", 64, [(0, 0), (0, 55)]),
])
def test_error_decomposition(name, rows_per_head, pairs):
    """Where the kernel's distance from the oracle comes from, on the
    sampled rows the workload test uses:
      bytes    the output the oracle's arithmetic (float64) gives from the
               kernel's own bytes and running maxima, against the oracle:
               the effect of bytes one code away (fp32 logits);
      fp32     the kernel's fp32 output before BF16 rounding, against that
               same float64 output from its bytes: the FP8 MFMA and fp32
               accumulation of P V and of the row sums;
      bf16     the BF16 output against the kernel's fp32 output.
    Each part stays below the tolerance, and they add up (in quadrature or
    less) to the total."""
    oc = _oc()
    w = workloads.WORKLOADS[name]
    log(f"[error parts] {name}")
    q, k, v = workloads.make_inputs(name, device="cuda")
    out = oc.attention(q, k, v)
    prep = oc.prepare(q, k, v)
    rows = np.array(workloads.sample_rows(w.S, rows_per_head, seed=w.seed))
    S = w.S
    for b, h in pairs:
        d = kernel_dump(prep, b, h, rows, out=out, out_f32=True)
        r = oracle_rows(q, k, v, b, h, rows, m_trace=d.m_used)
        ph = r["ph"]
        x = oracle.log2_logits(ph, rows, 1 / math.sqrt(128))
        check_max_trace(d.m_used, x, logit_error_bound(ph, rows, 1 / math.sqrt(128)))
        Mfin = d.m_used.max(axis=1)
        frame = np.exp2(d.m_used[:, np.arange(S) // 128] - Mfin[:, None])       # each key's tile weight in the final frame
        P = oracle.VALUES[d.codes] * frame
        from_bytes = float(ph.sv) * (P @ oracle.decode(ph.vc)) / P.sum(axis=1, keepdims=True)
        e_bytes = oracle.rel_l2(from_bytes, r["out"])
        e_fp32 = oracle.rel_l2(d.out_f32, from_bytes)
        e_bf16 = oracle.rel_l2(out_rows(out, b, h, rows), d.out_f32)
        e_tot = oracle.rel_l2(out_rows(out, b, h, rows), r["out"])
        per_row = np.linalg.norm(from_bytes - r["out"], axis=1) / np.linalg.norm(r["out"], axis=1)
        log(f"  ({b},{h}) total {e_tot:.2e} = bytes {e_bytes:.2e} (worst row {per_row.max():.2e}) + fp32 {e_fp32:.2e} "
            f"+ bf16 {e_bf16:.2e}")
        assert max(e_bytes, e_fp32, e_bf16) <= TOL
        assert e_tot <= e_bytes + e_fp32 + e_bf16 + 1e-12
