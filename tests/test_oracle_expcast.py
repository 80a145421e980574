"""Pins for the ExpCast byte map of the oracle against the figures of the
VC-Attention write-up (section "ExpCast-FP8"), reproduced here from closed
forms that do not go through the oracle's code."""
import json
import math
import os

import numpy as np

import oracle
from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "expcast_page_figures.json")) as f:
    PAGE = json.load(f)


def _rne(y):
    """round half to even for a Python float"""
    return round(y)


def analytic_pieces(beta):
    """Within one binade write v = 2^(e+u), u in [0,1). The ExpCast byte is
    8(e+7) + A(u) with A(u) = rne(8u + beta); the exp-then-cast byte is
    8(e+7) + B(u) with B(u) = rne(8(2^u - 1)). Both are step functions of u;
    return the pieces (u0, u1, A, B) between their breakpoints."""
    bps = {0.0, 1.0}
    for j in range(-1, 9):
        ua = (j + 0.5 - beta) / 8.0
        if 0 < ua < 1:
            bps.add(ua)
        ub = math.log2(1.0 + (j + 0.5) / 8.0)
        if 0 < ub < 1:
            bps.add(ub)
    bps = sorted(bps)
    pieces = []
    for u0, u1 in zip(bps[:-1], bps[1:]):
        um = 0.5 * (u0 + u1)
        pieces.append((u0, u1, _rne(8 * um + beta), _rne(8 * (2 ** um - 1))))
    return pieces


def analytic_agreement(beta):
    return sum(u1 - u0 for u0, u1, a, b in analytic_pieces(beta) if a == b)


def analytic_ratio_range(beta):
    """inf and sup over u of dec(ExpCast byte)/v = (1 + A(u)/8) / 2^u."""
    lo, hi = math.inf, -math.inf
    for u0, u1, a, _ in analytic_pieces(beta):
        hi = max(hi, (1 + a / 8) / 2 ** u0)
        lo = min(lo, (1 + a / 8) / 2 ** u1)
    return lo, hi


def tv_bound(lo, hi):
    """Largest total variation between p ~ w and p' ~ w*rho with rho in
    [lo, hi]: (sqrt(r)-1)/(sqrt(r)+1), r = hi/lo (two-point worst case)."""
    r = math.sqrt(hi / lo)
    return (r - 1) / (r + 1)


def test_closed_form_agreement_matches_page_figure():
    a = analytic_agreement(PAGE["beta"])
    assert abs(100 * a - PAGE["agreement_percent"]) < 0.05, a
    # neighbouring readings do not reproduce the figure: this pins the
    # rounding (nearest, not floor) and the sign/size of beta.
    assert abs(100 * analytic_agreement(0.0) - PAGE["agreement_percent"]) > 20
    assert abs(100 * analytic_agreement(+0.35) - PAGE["agreement_percent"]) > 20
    # floor rounding = rne(y - 0.5) everywhere except ties
    assert abs(100 * analytic_agreement(PAGE["beta"] - 0.5) - PAGE["agreement_percent"]) > 10
    # and every piece is at most one code apart
    assert max(abs(a - b) for _, _, a, b in analytic_pieces(PAGE["beta"])) == PAGE["max_code_distance"]


def test_closed_form_tv_bound_matches_page_figure():
    lo, hi = analytic_ratio_range(PAGE["beta"])
    assert abs(lo - 0.92900) < 5e-5 and abs(hi - 1.07453) < 5e-5
    b = tv_bound(lo, hi)
    assert round(100 * b, 2) == PAGE["tv_bound_percent"]


def test_oracle_codes_agree_with_closed_form_on_uniform_grid():
    """Oracle ExpCast bytes vs oracle exp-then-cast bytes on a fine uniform
    grid of log2 values across the normal binades: the share of equal bytes
    must equal the closed-form measure, and never differ by more than 1."""
    n = 1 << 20
    u = (np.arange(n) + 0.5) / n                  # one binade, midpoints
    x = np.concatenate([u + e for e in range(-14, 0)])   # x - M in [-14, 0): codes 8..120
    x = x[None, :]
    M = np.zeros(1, dtype=np.int64)
    c = oracle.expcast_codes(x, M)
    ce = oracle.exp_cast_codes(x, M)
    assert ce.min() >= 8
    agree = (c == ce).mean()
    assert abs(agree - analytic_agreement(PAGE["beta"])) < 2e-5
    assert np.abs(c.astype(int) - ce.astype(int)).max() == 1


def test_codes_are_one_fma_plus_round():
    """code = clamp(rne(8(x-M) + 120 + beta), 0, 126): the largest weight of a
    row lands in codes 112..120 and dec(120) = 256 = 2^8 * p_max-bound."""
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, (64, 500))
    M = oracle.bitaligned_row_max(x)
    assert np.all(M >= x.max(axis=1)) and np.all(M - 1 < x.max(axis=1))
    c = oracle.expcast_codes(x, M)
    top = c.max(axis=1)
    assert top.min() >= 112 and top.max() <= 120
    assert e4m3.VALUES[120] == 256.0
    # shift-equivariance: adding an integer n to x and M leaves the bytes alone
    for n in (-3, 1, 7):
        assert np.array_equal(oracle.expcast_codes(x + n, M + n), c)
    # weights below about 2^-15 of the row max underflow to code 0
    assert oracle.expcast_codes(np.array([[0.0, -15.1]]), np.array([0]))[0, 1] == 0


def test_row_tv_within_page_bound_on_attention_rows():
    import workloads
    q, k, v = workloads.make_inputs("s1024_h2")
    lo, hi = analytic_ratio_range(PAGE["beta"])
    bound = tv_bound(lo, hi)
    for h in range(2):
        qh, kh, vh = (t[0, :, h].double().numpy() for t in (q, k, v))
        ph = oracle.prepare_head(qh, kh, vh)
        rows = np.arange(0, 1024, 4)
        x = oracle.log2_logits(ph, rows, 1 / math.sqrt(128))
        M = oracle.bitaligned_row_max(x)
        c = oracle.expcast_codes(x, M)
        tv = oracle.row_total_variation(c, x)
        p = np.exp2(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        tail = np.where((x - M[:, None]) < -14, p, 0).sum(axis=1)   # exp byte would be subnormal
        assert np.all(tv <= bound + 2 * tail + 1e-12)
        assert 0.008 < tv.mean() < 0.02          # pages: mean 1.6% on real rows
        ce = oracle.exp_cast_codes(x, M)
        assert abs((c == ce).mean() - PAGE["agreement_percent"] / 100) < 0.005


def test_tv_bound_is_reached_by_two_level_row():
    """A row whose entries sit where dec(byte)/v is smallest or largest gets a
    TV close to the bound (so the oracle's bytes realise the page's bound)."""
    beta = PAGE["beta"]
    pieces = analytic_pieces(beta)
    lo, hi = analytic_ratio_range(beta)
    # u just below a breakpoint where the ratio is lowest / just at one where it is highest
    u_lo = min(pieces, key=lambda p: (1 + p[2] / 8) / 2 ** p[1])[1] - 1e-9
    u_hi = max(pieces, key=lambda p: (1 + p[2] / 8) / 2 ** p[0])[0] + 1e-9
    r = math.sqrt(hi / lo)
    t = 1 / (1 + r)                              # worst-case softmax mass at the high ratio
    n = 40000
    w_hi, w_lo = 2.0 ** u_hi, 2.0 ** u_lo
    n_hi = int(round(t * n * w_lo / (w_hi * (1 - t) + t * w_lo)))
    x = np.concatenate([np.full(n_hi, u_hi - 3.0), np.full(n - n_hi, u_lo - 3.0)])[None, :]
    M = np.array([0])
    c = oracle.expcast_codes(x, M)
    tv = oracle.row_total_variation(c, x)[0]
    assert tv <= tv_bound(lo, hi) + 1e-6
    assert tv > tv_bound(lo, hi) - 2e-4
