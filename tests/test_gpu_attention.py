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
from gpu_util import head64, log, oracle_rows, out_rows

pytestmark = pytest.mark.gpu

TOL = 5e-3
# oracle byte path -> the kernel's name for it
KERNEL_WEIGHTS = {"expcast": "expcast", "exp_cast": "exp_fp8"}


def _oc():
    import bit_fp8_attention_block_amd as oc
    return oc


def logit_error_bound(ph, rows, tau):
    """Worst-case difference between the kernel's logit and the exact one.
    The FP8 MFMA does not sum its 128 products to fp32 accuracy: measured on
    gfx950 against exact sums (8192 trials of random codes, and of small
    codes beside one dominant product), its error stayed within 2^-11.3 of
    the largest product's magnitude; the bound allows 2^-10 of the largest
    possible product, max|q| * max|k|. On top of that, fp32 rounding of the
    sum (128 * 2^-24 * sum |products|) and of the three scale products and
    the FMA (a few ulp of the logit)."""
    qd = np.abs(oracle.decode(ph.qc[np.asarray(rows)]))
    kd = np.abs(oracle.decode(ph.kc))
    sqr = ph.sq[np.asarray(rows) // 128].astype(np.float64)
    skk = ph.sk[np.arange(ph.S) // 128].astype(np.float64)
    scale = (tau / math.log(2)) * (sqr[:, None] * skk[None, :])
    mag = scale * (qd @ kd.T)
    top = scale * np.outer(qd.max(axis=1), kd.max(axis=1))
    return mag * (128 * 2.0 ** -24) + mag * 2.0 ** -20 + top * 2.0 ** -10


def check_max_trace(kernel_trace, own, x, bound, order="mid"):
    """The kernel's running max per tile must match the oracle's, except where
    a tile's largest logit lies within the kernel's logit error bound of an
    integer:
    there the first divergence must be exactly one, at such a tie."""
    nT = kernel_trace.shape[1]
    tiles = oracle.key_tile_order(nT) if order == "mid" else list(range(nT))
    S = x.shape[1]
    bad_rows = np.nonzero((kernel_trace != own).any(axis=1))[0]
    for i in bad_rows:
        for t in tiles:
            if kernel_trace[i, t] != own[i, t]:
                sl = slice(t * 128, min(S, t * 128 + 128))
                xm = x[i, sl].max()
                assert abs(int(kernel_trace[i, t]) - int(own[i, t])) == 1, (i, t)
                assert abs(xm - round(xm)) <= bound[i, sl].max(), (i, t, xm, bound[i, sl].max())
                break
    return len(bad_rows)


def _compare(q, k, v, out, pairs, rows, budget=0.0, tol=TOL, label="", order="mid", prep=None, weights="expcast",
             k_smooth=False, v_smooth=False, tau=None):
    """rel-L2 of the kernel's rows against the single-pass oracle. With a
    prepared workspace, the oracle replays the running-max decisions the
    kernel made (read back through the debug dump), after checking that each
    of them agrees with the oracle's own or is a rounding tie at an integer."""
    errs, two = [], []
    nflip = 0
    for b, h in pairs:
        m_trace = None
        if prep is not None:
            oc = _oc()
            _, m_used, _ = oc.debug_pcodes(prep, b, h, with_codes=False, weights=KERNEL_WEIGHTS[weights])
            m_trace = m_used[torch.as_tensor(rows, device=m_used.device)].cpu().numpy()
            own = oracle_rows(q, k, v, b, h, rows, budget=budget, tau=tau, order=order, weights=weights,
                              k_smooth=k_smooth, v_smooth=v_smooth)
            t = tau if tau else 1 / math.sqrt(128)
            x = oracle.log2_logits(own["ph"], rows, t)
            nflip += check_max_trace(m_trace, own["m_trace"], x, logit_error_bound(own["ph"], rows, t), order)
        r = oracle_rows(q, k, v, b, h, rows, budget=budget, tau=tau, order=order, m_trace=m_trace, weights=weights,
                        k_smooth=k_smooth, v_smooth=v_smooth)
        got = out_rows(out, b, h, rows)
        e = oracle.rel_l2(got, r["out"])
        errs.append(e)
        r2 = oracle.expcast_attention_head(head64(q, b, h), head64(k, b, h), head64(v, b, h), tau=tau, rows=rows,
                                           ph=r["ph"], weights=weights)
        two.append(oracle.rel_l2(got, r2["out"]))
        assert np.isfinite(got).all()
        assert e <= tol, (label, b, h, e)
    log(f"  {label}: rel-L2 vs oracle (single-pass form) max {max(errs):.2e}; vs two-pass form max {max(two):.2e}"
        + (f"; rows with a tie-broken max {nflip}" if prep is not None else ""))
    return errs


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
    prep = oc.prepare(q, k, v)
    tau = 1 / math.sqrt(128)
    for b in range(B):
        for h in range(H):
            codes, m_used, out = oc.debug_pcodes(prep, b, h)
            torch.cuda.synchronize()
            codes, m_used = codes.cpu().numpy(), m_used.cpu().numpy()
            ph = oracle.prepare_head(head64(q, b, h), head64(k, b, h), head64(v, b, h))
            x = oracle.log2_logits(ph, np.arange(S), tau)
            tiles = np.arange(S) // 128
            Mk = m_used[:, tiles]                      # running max used for each (row, key)
            assert (Mk > -(1 << 29)).all(), "every tile must have been visited"
            want = oracle.expcast_codes(x, Mk)
            diff = np.abs(codes.astype(int) - want.astype(int))
            agree = (diff == 0).mean()
            log(f"  (b={b},h={h}) byte agreement {agree:.6f}, max diff {diff.max()}")
            assert agree >= 0.999 and diff.max() <= 1
            # the final running max is the bit-aligned row max, except where the
            # row's largest logit lies within the logit error bound of an integer
            Mfinal = m_used.max(axis=1)
            Mo = oracle.bitaligned_row_max(x)
            bad = np.nonzero(Mfinal != Mo)[0]
            xmax = x.max(axis=1)
            bound = logit_error_bound(ph, np.arange(S), tau) if len(bad) else None
            for i in bad:
                gap = abs(xmax[i] - round(xmax[i]))
                log(f"  row {i}: kernel M {Mfinal[i]} oracle M {Mo[i]} (max logit {xmax[i]:.9f})")
                assert abs(int(Mfinal[i]) - int(Mo[i])) == 1 and gap <= bound[i].max()
            # the dumped output equals the oracle too
            r = oracle.expcast_attention_online(head64(q, b, h), head64(k, b, h), head64(v, b, h), ph=ph)
            e = oracle.rel_l2(out_rows(out, b, h, np.arange(S)), r["out"])
            assert e <= TOL, e


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


def test_deterministic_and_graph_replays():
    """The prepare graph is replayed on every call; eager work in between must
    not disturb it and every replay must give the same bits."""
    oc = _oc()
    q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=4096, H=4)
    ref = oc.attention(q, k, v).clone()
    for i in range(4):
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
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
