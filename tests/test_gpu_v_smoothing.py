"""V-Smooth block means against the oracle: the bf16 block means, the
residual codes and scale, the scaled means in the kernel's operand order and,
with repair, the residual energies and selection, bit-exact; attention with the
means added back per key tile within 5e-3 of the oracle; lower error than the
plain path on values with a per-channel bias."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import WsView, head64, log, out_rows
from test_gpu_attention import _compare

pytestmark = pytest.mark.gpu


def _oc():
    import bit_fp8_attention_block_amd as oc
    return oc


def _biased_values(B, S, H, seed, dtype=torch.bfloat16):
    """q, k ~ N(0,1); v ~ N(0,1) plus an N(0, 5^2) bias per (head, channel)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, H, 128, generator=g)
    k = torch.randn(B, S, H, 128, generator=g)
    v = torch.randn(B, S, H, 128, generator=g) + 5.0 * torch.randn(1, 1, H, 128, generator=g)
    return tuple(t.to(dtype).cuda() for t in (q, k, v))


@pytest.mark.parametrize("case", ["s1024_h2", "ragged_fp16", "biased", "repair"])
def test_smoothed_value_prepare_bit_exact(case):
    oc = _oc()
    log(f"[v-smooth prepare] case={case}")
    budget = None
    if case == "s1024_h2":
        q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    elif case == "ragged_fp16":
        q, k, v = workloads.make_inputs("b2_s70000_h40_fp16", device="cuda", S=300, H=3)
    elif case == "biased":
        q, k, v = _biased_values(1, 700, 2, seed=4)
    else:
        q, k, v = workloads.make_inputs("s8192_h8", device="cuda", S=1500, H=2)
        budget = 0.02
    prep = oc.prepare(q, k, v, budget=budget, v_smooth=True)
    torch.cuda.synchronize()
    w = WsView(prep)
    B, S, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            vh = head64(v, b, h)
            ph = oracle.prepare_head(head64(q, b, h), head64(k, b, h), vh, budget=budget or 0.0, v_smooth=True)
            mu_bits = (ph.vmean.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            assert np.array_equal(w.vmu(b, h), mu_bits), (b, h, "block means")
            assert np.array_equal(w.vcodes(b, h), ph.vc), (b, h, "residual codes")
            s, _ = w.sv(b, h)
            assert s == ph.sv, (b, h, "residual scale")
            if budget:
                rp = ph.repair
                assert np.array_equal(w.energy(b, h), rp.energy) or np.allclose(w.energy(b, h), rp.energy,
                                                                                  rtol=1e-14, atol=0)
                assert np.array_equal(w.sel(b, h, rp.k), rp.sel), (b, h, "selection")
                assert np.array_equal(w.rcodes(b, h, rp.k), rp.rc), (b, h, "repair codes")
                assert w.sr(b, h)[0] == rp.sr


@pytest.mark.parametrize("name", ["s8192_h8", "biased"])
def test_smoothed_value_attention_matches_oracle(name):
    oc = _oc()
    log(f"[v-smooth attention] {name}")
    if name == "biased":
        q, k, v = _biased_values(1, 4000, 2, seed=5)
        rows, pairs = np.arange(0, 4000, 9), [(0, 0), (0, 1)]
    else:
        q, k, v = workloads.make_inputs(name, device="cuda")
        rows, pairs = np.array(workloads.sample_rows(8192, 256, seed=2)), [(0, 0), (0, 6)]
    out = oc.attention(q, k, v, v_smooth=True)
    prep = oc.prepare(q, k, v, v_smooth=True)
    torch.cuda.synchronize()
    _compare(q, k, v, out, pairs, rows, label=name + " V-Smooth", prep=prep, v_smooth=True)


@pytest.mark.parametrize("S", [1, 5, 130, 300, 700, 1000, 1500, 2100, 4200])
def test_smoothed_value_attention_ragged_batches(S):
    """The mean term is added sixteen key tiles at a time; these lengths give
    1, 1, 2, 3, 6, 8, 12, 17 and 33 tiles, so the last batch is partial (down
    to one tile after full ones) in both wave groups, and the last tile is
    ragged."""
    oc = _oc()
    log(f"[v-smooth ragged] S={S}")
    q, k, v = _biased_values(1, S, 2, seed=11 + S)
    out = oc.attention(q, k, v, v_smooth=True)
    prep = oc.prepare(q, k, v, v_smooth=True)
    torch.cuda.synchronize()
    _compare(q, k, v, out, [(0, 0), (0, 1)], np.arange(S), label=f"V-Smooth S={S}", prep=prep, v_smooth=True)


def test_smoothed_value_attention_full_size_sampled():
    """S=73397, H=56 (574 key tiles: the last batch holds fourteen), sampled rows of
    three heads, including the ragged tail."""
    oc = _oc()
    name = "s73397_h56"
    w = workloads.WORKLOADS[name]
    log(f"[v-smooth full size] {name}")
    q, k, v = workloads.make_inputs(name, device="cuda")
    out = oc.attention(q, k, v, v_smooth=True)
    prep = oc.prepare(q, k, v, v_smooth=True)
    torch.cuda.synchronize()
    rows = np.array(workloads.sample_rows(w.S, 64, seed=w.seed))
    _compare(q, k, v, out, [(0, 0), (0, 29), (0, 55)], rows, label=name + " V-Smooth", prep=prep, v_smooth=True)


def test_smoothed_value_attention_with_repair_matches_oracle():
    oc = _oc()
    q, k, v = _biased_values(1, 2000, 2, seed=6)
    out = oc.attention_v_repair(q, k, v, 0.01, v_smooth=True)
    prep = oc.prepare_v_repair(q, k, v, 0.01, v_smooth=True)
    torch.cuda.synchronize()
    _compare(q, k, v, out, [(0, 0), (0, 1)], np.arange(0, 2000, 3), budget=0.01, label="V-Smooth + repair",
             prep=prep, v_smooth=True)


def test_smoothing_lowers_value_error_on_channel_biased_values():
    """The values the kernel multiplies by (block mean + sv * residual code,
    read back from the workspace) against the input values: removing a
    per-channel bias shrinks the E4M3 range, so the error drops sharply. The
    attention output improves too, down to the BF16 output rounding."""
    oc = _oc()
    q, k, v = _biased_values(1, 4096, 2, seed=7)
    prep_s = oc.prepare(q, k, v, v_smooth=True)
    prep_p = oc.prepare(q, k, v)
    plain = oc.attention(q, k, v)
    smooth = oc.attention(q, k, v, v_smooth=True)
    torch.cuda.synchronize()
    ws, wp = WsView(prep_s), WsView(prep_p)
    rows = np.arange(0, 4096, 16)
    for h in range(2):
        vh = head64(v, 0, h)
        rec_p = float(wp.sv(0, h)[0]) * oracle.decode(wp.vcodes(0, h))
        mu = (ws.vmu(0, h).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rec_s = mu[np.arange(4096) // 128] + float(ws.sv(0, h)[0]) * oracle.decode(ws.vcodes(0, h))
        ev0, ev1 = oracle.rel_l2(rec_p, vh), oracle.rel_l2(rec_s, vh)
        exact = oracle.exact_attention_head(head64(q, 0, h), head64(k, 0, h), vh, rows=rows)
        e0 = oracle.rel_l2(out_rows(plain, 0, h, rows), exact)
        e1 = oracle.rel_l2(out_rows(smooth, 0, h, rows), exact)
        log(f"  (h={h}) value rel-L2: plain {ev0:.5f}, V-Smooth {ev1:.5f}; "
            f"output vs exact: plain {e0:.5f}, V-Smooth {e1:.5f}")
        assert ev1 < 0.5 * ev0
        assert e1 < e0


def test_prepared_call_follows_the_workspace_setting():
    oc = _oc()
    q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    full = oc.attention(q, k, v, v_smooth=True)
    prep = oc.prepare(q, k, v, v_smooth=True)
    other = oc.prepare(q, k, v)                       # same plan, smoothing off again
    a = oc.attention_prepared(prep)
    b = oc.attention_prepared(other)
    plain = oc.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, full) and torch.equal(b, plain) and not torch.equal(a, b)


@pytest.mark.parametrize("S,fp16", [(300, False), (1000, True)])
def test_all_options_together_match_oracle(S, fp16):
    """The comparison byte path with K-mean smoothing, V-Smooth and repair in
    one call (three and eight key tiles, bf16 and fp16 inputs)."""
    oc = _oc()
    log(f"[all options] S={S} fp16={fp16}")
    q, k, v = _biased_values(1, S, 2, seed=40 + S, dtype=torch.float16 if fp16 else torch.bfloat16)
    k = k + 2.0   # a shared key offset for the smoothing to remove
    opts = dict(weights="exp_fp8", k_smooth=True, v_smooth=True)
    out = oc.attention_v_repair(q, k, v, 0.02, **opts)
    prep = oc.prepare_v_repair(q, k, v, 0.02, k_smooth=True, v_smooth=True)
    torch.cuda.synchronize()
    _compare(q, k, v, out, [(0, 0), (0, 1)], np.arange(S), budget=0.02, label=f"all options S={S}", prep=prep,
             weights="exp_cast", k_smooth=True, v_smooth=True)
