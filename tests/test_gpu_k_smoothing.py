"""K-mean smoothing in the prepare step against the oracle: the mean key
(fp32) and the K codes and scales of fp32(k - kbar) bit-exact, Q and V
untouched; attention on the smoothed keys within 5e-3 of the oracle; and on
keys with a per-channel bias, a lower error against exact attention than
without smoothing."""
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


@pytest.mark.parametrize("case", ["s1024_h2", "ragged_fp16", "strided", "tiny"])
def test_smoothed_prepare_bit_exact(case):
    oc = _oc()
    log(f"[k-smooth prepare] case={case}")
    if case == "s1024_h2":
        q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    elif case == "ragged_fp16":
        q, k, v = workloads.make_inputs("b2_s70000_h40_fp16", device="cuda", S=300, H=3)
    elif case == "strided":
        qkv = torch.randn(2, 520, 3, 2, 128, device="cuda").mul_(3).add_(2).to(torch.bfloat16)
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    else:
        q, k, v = workloads.random_qkv(1, 1, 1, seed=3, device="cuda")
    prep = oc.prepare(q, k, v, k_smooth=True)
    plain = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    w, w0 = WsView(prep), WsView(plain)
    B, S, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            qh, kh, vh = head64(q, b, h), head64(k, b, h), head64(v, b, h)
            ph = oracle.prepare_head(qh, kh, vh, k_smooth=True)
            assert np.array_equal(w.kmean(b, h), oracle.key_mean(kh)), (b, h, "mean key")
            assert np.array_equal(w.kcodes(b, h), ph.kc), (b, h, "k codes")
            assert np.array_equal(w.sk(b, h), ph.sk), (b, h, "k scales")
            assert np.array_equal(w.qcodes(b, h), w0.qcodes(b, h)) and np.array_equal(w.sq(b, h), w0.sq(b, h))
            assert np.array_equal(w.vcodes(b, h), w0.vcodes(b, h))


@pytest.mark.parametrize("name,rows_per_head,pairs", [
    ("s8192_h8", 256, [(0, 0), (0, 3)]),
    ("b2_s70000_h40_fp16", 64, [(0, 0), (1, 39)]),
])
def test_smoothed_attention_matches_oracle(name, rows_per_head, pairs):
    oc = _oc()
    w = workloads.WORKLOADS[name]
    log(f"[k-smooth attention] {name}")
    q, k, v = workloads.make_inputs(name, device="cuda")
    out = oc.attention(q, k, v, k_smooth=True)
    prep = oc.prepare(q, k, v, k_smooth=True)
    torch.cuda.synchronize()
    rows = np.array(workloads.sample_rows(w.S, rows_per_head, seed=w.seed))
    _compare(q, k, v, out, pairs, rows, label=name + " K-smoothed", prep=prep, k_smooth=True)


def test_smoothing_lowers_error_vs_exact_on_biased_keys():
    """fp16 workload with an N(0,3) per-channel bias on Q and K (S=4096, 2
    heads): relative L2 against exact float64 attention, with and without
    smoothing."""
    oc = _oc()
    q, k, v = workloads.make_inputs("b2_s70000_h40_fp16", device="cuda", S=4096, H=2)
    plain = oc.attention(q, k, v)
    smooth = oc.attention(q, k, v, k_smooth=True)
    torch.cuda.synchronize()
    rows = np.arange(0, 4096, 16)
    for b, h in ((0, 0), (1, 1)):
        exact = oracle.exact_attention_head(head64(q, b, h), head64(k, b, h), head64(v, b, h), rows=rows)
        e0 = oracle.rel_l2(out_rows(plain, b, h, rows), exact)
        e1 = oracle.rel_l2(out_rows(smooth, b, h, rows), exact)
        log(f"  (b={b},h={h}) rel-L2 vs exact: plain {e0:.4f}, K-smoothed {e1:.4f}")
        assert e1 < e0


def test_smoothing_switch_is_per_call():
    oc = _oc()
    q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    a = oc.attention(q, k, v)
    s = oc.attention(q, k, v, k_smooth=True)
    a2 = oc.attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, a2) and not torch.equal(a, s)
