"""Prepare kernels vs the oracle, bit-exact: Q/K block codes and scales, V
head codes and scale (after undoing the pack layouts), padding left zero."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import WsView, head64, log

pytestmark = pytest.mark.gpu


def _check_prepared(q, k, v, prep):
    w = WsView(prep)
    B, S, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            ph = oracle.prepare_head(head64(q, b, h), head64(k, b, h), head64(v, b, h))
            qc = w.qcodes(b, h)
            assert np.array_equal(qc[:S], ph.qc), (b, h, "q codes")
            assert not qc[S:].any(), "q padding rows must be zero"
            sq = w.sq(b, h)
            assert np.array_equal(sq[:len(ph.sq)], ph.sq), (b, h, "q scales")
            assert np.all(sq[len(ph.sq):] == 1.0)
            assert np.array_equal(w.kcodes(b, h), ph.kc), (b, h, "k codes")
            assert np.array_equal(w.sk(b, h), ph.sk), (b, h, "k scales")
            assert np.array_equal(w.vcodes(b, h), ph.vc), (b, h, "v codes")
            s, inv = w.sv(b, h)
            assert s == ph.sv, (b, h, "v scale")
            _, inv_o = oracle.quant_scale(np.abs(head64(v, b, h)).max())
            assert inv == inv_o
            # padding keys of the last tile are zero in both packs
            nT = w.L.n_ktiles
            if S % 128:
                from gpu_util import unpack_k, unpack_v
                n = nT * 16384
                kr = w._arr(w.L.kpack + w.bh(b, h) * n, np.uint8, n)
                assert not unpack_k(kr, nT * 128)[S:].any()
                assert not unpack_v(w.vraw(b, h), nT * 128)[S:].any()


@pytest.mark.parametrize("case", ["s1024_h2", "ragged_fp16", "strided", "tiny"])
def test_prepare_bit_exact(case):
    import bit_fp8_attention_block_amd as oc
    log(f"[prepare] case={case}")
    if case == "s1024_h2":
        q, k, v = workloads.make_inputs("s1024_h2", device="cuda")
    elif case == "ragged_fp16":
        q, k, v = workloads.make_inputs("b2_s70000_h40_fp16", device="cuda", S=300, H=3)
    elif case == "strided":
        qkv = torch.randn(2, 520, 3, 2, 128, device="cuda").mul_(3).to(torch.bfloat16)
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    else:
        q, k, v = workloads.random_qkv(1, 1, 1, seed=3, device="cuda")
    prep = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    _check_prepared(q, k, v, prep)


def test_prepare_extreme_ranges():
    """Blocks spanning the whole bf16 range, all-zero blocks, values that land
    on E4M3 subnormals and exact ties."""
    import bit_fp8_attention_block_amd as oc
    log("[prepare] extreme ranges")
    S, H = 512, 2
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(1, S, H, 128, device="cuda", generator=g)
    x = x * torch.exp2(torch.randint(-30, 30, (1, S, H, 1), device="cuda", generator=g).float())
    q = x.to(torch.bfloat16)
    k = (x * 1e-3).to(torch.bfloat16)
    k[:, 128:256] = 0           # an all-zero block: scale 1, codes 0
    v = torch.randn(1, S, H, 128, device="cuda", generator=g).to(torch.bfloat16)
    v[0, 5, 0, :] = 1e4          # one huge value sets the head scale, most codes go subnormal
    prep = oc.prepare(q, k, v)
    torch.cuda.synchronize()
    _check_prepared(q, k, v, prep)


def test_prepare_tiny_blocks_take_the_unit_scale():
    """Blocks (and a whole head of V) whose amax lies below 2^-100 take the
    unit scale and codes 0 (0x80 for negative values), while a block whose
    amax is 2^-100 itself and one just above take their regular scales."""
    import bit_fp8_attention_block_amd as oc
    log("[prepare] tiny blocks")
    S, H = 640, 2
    g = torch.Generator().manual_seed(12)
    x = torch.randn(1, S, H, 128, generator=g)
    q = x.clone()
    q[:, 0:128] *= 2.0 ** -110          # below the floor: unit scale
    q[:, 128:256] *= 2.0 ** -102        # |x| up to ~2^-100: straddles the floor, some blocks each way
    k = x.flip(1).clone()
    k[:, 256:384] *= 2.0 ** -120
    blk = k[:, 384:512]
    k[:, 384:512] = blk / blk.abs().amax(dim=(0, 1, 3), keepdim=True) * 2.0 ** -100   # amax exactly 2^-100: regular
    v = torch.randn(1, S, H, 128, generator=g)
    v[:, :, 1] *= 2.0 ** -115           # the whole of head 1 is below the floor
    q, k, v = (t.to(torch.bfloat16).cuda() for t in (q, k, v))
    prep = oc.prepare(q, k, v)
    out = oc.attention(q, k, v)
    torch.cuda.synchronize()
    _check_prepared(q, k, v, prep)
    w = WsView(prep)
    assert np.all(w.sq(0, 0)[0] == 1.0) and np.all(w.sk(0, 0)[2] == 1.0)
    assert w.sk(0, 0)[3] != 1.0
    assert w.sv(0, 1)[0] == 1.0 and not (w.vcodes(0, 1) & 0x7F).any()
    assert (w.vcodes(0, 1) == 0x80).any()
    # head 1's values all count as zero: its output is zero
    assert torch.isfinite(out.float()).all()
    assert not out[0, :, 1].float().abs().max().item()


def test_prepare_fp16_extremes():
    """fp16 inputs at the ends of their range: values up to 65504, blocks of
    fp16 subnormals (down to 2^-24), exact zeros and a head of V made of
    subnormals only. Codes and scales bit-exact; the output finite and within
    the usual tolerance of the oracle."""
    import bit_fp8_attention_block_amd as oc
    from gpu_util import compare
    log("[prepare] fp16 extremes")
    S, H = 700, 2
    g = torch.Generator().manual_seed(21)
    x = torch.randn(1, S, H, 128, generator=g)
    q = (x * 20000.0).clamp(-65504, 65504)
    q[0, 3, 0, 7] = 65504.0                                   # the largest finite fp16
    k = x.flip(1) * 3.0
    k[:, 128:256] = torch.randint(-1023, 1024, (1, 128, H, 128), generator=g).float() * 2.0 ** -24  # subnormals
    k[:, 256:384, 1] = 0.0
    v = torch.randn(1, S, H, 128, generator=g)
    v[:, :, 1] = torch.randint(-1023, 1024, (1, S, 128), generator=g).float() * 2.0 ** -24          # head 1: subnormal V
    q, k, v = (t.to(torch.float16).cuda() for t in (q, k, v))
    assert torch.isfinite(q.float()).all() and (k[:, 128:256].float().abs().max() < 2.0 ** -14)
    prep = oc.prepare(q, k, v)
    out = oc.attention(q, k, v)
    torch.cuda.synchronize()
    _check_prepared(q, k, v, prep)
    assert torch.isfinite(out.float()).all()
    compare(q, k, v, out, [(0, 0), (0, 1)], np.arange(S), label="fp16 extremes", prep=prep)
