"""Seeded synthetic inputs for the FP8 ExpCast attention path.

This module only draws random tensors. It holds none of the method's
arithmetic: it is shared by the tests, the benchmark and the smoke check so
that the oracle and the GPU library see identical input bits.

The recipes stand in for the activations the pages measured on (real
MiniMax-H3 and Wan2.2 captures, which are not available). Shapes follow the
pages: head dim 128, the MiniMax-H3 shape S=73397 with 56 heads, and the
Wan2.2-14B shape of about 70K tokens with 40 heads. The value structure
follows the VC-Attention write-up ("V-Smooth" section): a few value tokens
carry outliers on a handful of channels, and those channels can persist
across heads.

Every tensor is [B, S, H, 128], drawn in float32 from a torch.Generator
seeded per workload, then rounded to nearest-even into bf16 or fp16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

D = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    dtype: torch.dtype
    qk_bias_var: float      # variance of the per-(head, channel) bias added to Q and K
    qk_lognormal_sigma: float  # sigma of the per-(head, channel) log-normal scale of Q and K (0 = none)
    v_kind: str             # "normal" or "student_t3"
    v_base_scale: float
    outlier_frac: float     # fraction of value tokens that carry outliers (per (b, h))
    outlier_channels: int
    outlier_gain: float
    outliers_shared_across_heads: bool
    budgets: tuple
    seed: int


# The five workloads: a small case the oracle runs in full, three growing
# video-DiT-like shapes, and the Wan2.2-like fp16 shape with heavy-tailed V.
WORKLOADS = {
    "s1024_h2": Workload("s1024_h2", 1, 1024, 2, torch.bfloat16, 0.0, 0.0, "normal", 1.0,
                         0.0, 0, 1.0, False, (0.0,), 1),
    "s8192_h8": Workload("s8192_h8", 1, 8192, 8, torch.bfloat16, 2.0, 0.0, "normal", 1.0,
                         0.01, 8, 20.0, False, (0.0, 0.005), 2),
    "s32768_h14": Workload("s32768_h14", 1, 32768, 14, torch.bfloat16, 2.0, 0.0, "normal", 1.0,
                           0.01, 8, 20.0, True, (0.0, 0.005, 0.01), 3),
    "s73397_h56": Workload("s73397_h56", 1, 73397, 56, torch.bfloat16, 2.0, 0.5, "normal", 1.0,
                           0.01, 8, 20.0, False, (0.0, 0.005, 0.01, 0.02), 4),
    "b2_s70000_h40_fp16": Workload("b2_s70000_h40_fp16", 2, 70000, 40, torch.float16, 3.0, 0.0,
                                   "student_t3", 0.5, 0.02, 16, 30.0, False, (0.005,), 5),
}

HEADLINE = "s73397_h56"


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _outlier_mask_gain(B, S, H, frac, nch, gain, shared, gen, device):
    """Multiplicative gain tensor [B,S,H,D]: 1 everywhere except `gain` on the
    outlier (token, channel) pairs. ceil(frac*S) distinct tokens per (b, h)
    (per b when shared across heads), each with `nch` distinct channels."""
    g = torch.ones((B, S, H, D), device=device, dtype=torch.float32)
    n_tok = int(math.ceil(frac * S))
    if n_tok == 0 or nch == 0:
        return g
    groups = [(b, None) for b in range(B)] if shared else [(b, h) for b in range(B) for h in range(H)]
    for b, h in groups:
        toks = torch.randperm(S, generator=gen, device=device)[:n_tok]
        chans = torch.rand((n_tok, D), generator=gen, device=device).argsort(dim=1)[:, :nch]
        if h is None:
            for hh in range(H):
                g[b, toks.unsqueeze(1), hh, chans] = gain
        else:
            g[b, toks.unsqueeze(1), h, chans] = gain
    return g


def make_inputs(w: Workload | str, device="cpu", S=None, H=None, B=None, seed=None):
    """Return (q, k, v) as [B,S,H,128] tensors in the workload's dtype.

    S, H, B and seed may be overridden to get a smaller tensor with the same
    value structure (used for ragged-size and edge-case tests).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    S = w.S if S is None else S
    H = w.H if H is None else H
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (B, S, H, D)
    # Draw order is fixed: Q noise, K noise, Q structure, K structure, V, V outliers.
    qn = _randn(shape, gen, device)
    kn = _randn(shape, gen, device)

    def structure(x):
        if w.qk_lognormal_sigma > 0:
            x = x * torch.exp(w.qk_lognormal_sigma * _randn((1, 1, H, D), gen, device))
        if w.qk_bias_var > 0:
            x = x + math.sqrt(w.qk_bias_var) * _randn((1, 1, H, D), gen, device)
        return x

    q = structure(qn)
    k = structure(kn)
    del qn, kn
    if w.v_kind == "normal":
        v = w.v_base_scale * _randn(shape, gen, device)
    elif w.v_kind == "student_t3":
        z = _randn(shape, gen, device)
        chi2 = sum(_randn(shape, gen, device) ** 2 for _ in range(3))
        v = w.v_base_scale * z / torch.sqrt(chi2 / 3.0)
        del z, chi2
    else:
        raise ValueError(w.v_kind)
    if w.outlier_frac > 0:
        v = v * _outlier_mask_gain(B, S, H, w.outlier_frac, w.outlier_channels, w.outlier_gain,
                                   w.outliers_shared_across_heads, gen, device)
    return q.to(w.dtype), k.to(w.dtype), v.to(w.dtype)


def random_qkv(B, S, H, dtype=torch.bfloat16, seed=0, device="cpu", scale=1.0):
    """Plain i.i.d. N(0, scale^2) inputs for edge-case tests."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (B, S, H, D)
    return tuple((scale * _randn(shape, gen, device)).to(dtype) for _ in range(3))


def sample_rows(S, n, seed=0):
    """Deterministic sample of n distinct query rows in [0, S), always
    including the first row, the last row (tail tile) and a row of the last
    full 128-block."""
    if n >= S:
        return list(range(S))
    gen = torch.Generator().manual_seed(1000 + seed)
    pick = set(torch.randperm(S, generator=gen)[: max(0, n - 3)].tolist())
    pick.update({0, S - 1, max(0, (S // 128) * 128 - 1)})
    return sorted(pick)[:n] if len(pick) > n else sorted(pick)
