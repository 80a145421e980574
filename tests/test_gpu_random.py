"""Seeded random configurations against the oracle: batch, length, heads,
input dtype, memory layout (contiguous, [S,H,128], a view of a fused qkv
tensor), softmax scale, repair budget and the byte-path and smoothing
options are drawn per case, and the output must stay within 5e-3 of the
single-pass oracle on every checked row, with the kernel's running-max
decisions replayed as in the other attention tests."""
import math

import numpy as np
import pytest
import torch

import workloads
from gpu_util import log
from test_gpu_attention import _compare

pytestmark = pytest.mark.gpu

N_CASES = 48


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    return dict(
        B=int(r.integers(1, 3)),
        S=int(r.choice([int(r.integers(1, 300)), int(r.integers(300, 1500)), int(r.integers(1500, 3000))])),
        H=int(r.integers(1, 4)),
        fp16=bool(r.integers(0, 2)),
        layout=str(r.choice(["contiguous", "three_dim", "fused_qkv"])),
        scale=float(r.choice([0.0, 0.05, 0.12, 0.3, 1.0])),
        budget=float(r.choice([0.0, 0.0, 0.01, 0.05])),
        weights=str(r.choice(["expcast", "expcast", "exp_fp8"])),
        k_smooth=bool(r.integers(0, 3) == 0),
        v_smooth=bool(r.integers(0, 3) == 0),
        bias=float(r.choice([0.0, 1.5])),
    )


def _inputs(c, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.float16 if c["fp16"] else torch.bfloat16
    B = 1 if c["layout"] == "three_dim" else c["B"]
    shape = (B, c["S"], c["H"], 128)
    mk = lambda: torch.randn(*shape, generator=g) + c["bias"] * torch.randn(1, 1, c["H"], 128, generator=g)  # noqa: E731
    if c["layout"] == "fused_qkv":
        qkv = torch.stack([mk(), mk(), mk()], dim=3).to(dt).cuda()        # [B, S, H, 3, 128]
        return qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2]
    q, k, v = (mk().to(dt).cuda() for _ in range(3))
    if c["layout"] == "three_dim":
        return q[0], k[0], v[0]
    return q, k, v


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration_matches_oracle(seed):
    import bit_fp8_attention_block_amd as oc
    c = _case(seed)
    log(f"[random {seed}] {c}")
    q, k, v = _inputs(c, seed)
    opts = dict(weights=c["weights"], k_smooth=c["k_smooth"], v_smooth=c["v_smooth"])
    scale = c["scale"] or None
    if c["budget"] > 0:
        out = oc.attention_v_repair(q, k, v, c["budget"], softmax_scale=scale, **opts)
        prep = oc.prepare_v_repair(q, k, v, c["budget"], softmax_scale=scale, k_smooth=c["k_smooth"],
                                   v_smooth=c["v_smooth"])
    else:
        out = oc.attention(q, k, v, softmax_scale=scale, **opts)
        prep = oc.prepare(q, k, v, softmax_scale=scale, k_smooth=c["k_smooth"], v_smooth=c["v_smooth"])
    torch.cuda.synchronize()
    if q.dim() == 3:
        q, k, v, out = q[None], k[None], v[None], out[None]
    B, S, H, _ = q.shape
    rows = np.arange(S) if S <= 600 else np.array(workloads.sample_rows(S, 300, seed=seed))
    pairs = [(b, h) for b in range(B) for h in range(H)][:3]
    _compare(q, k, v, out, pairs, rows, budget=c["budget"], label=f"random {seed}", prep=prep,
             weights="exp_cast" if c["weights"] == "exp_fp8" else "expcast", k_smooth=c["k_smooth"],
             v_smooth=c["v_smooth"], tau=scale)
