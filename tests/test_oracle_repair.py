"""Pins for the oracle's V-residual repair (Open-VC news, section on ExpCast
and the move away from exponentials; product page, repair paragraph)."""
import math

import numpy as np
import pytest

import oracle
import workloads


def _head(name="s8192_h8", S=2048, h=0):
    q, k, v = workloads.make_inputs(name, S=S, H=1)
    return tuple(t[0, :, h].double().numpy() for t in (q, k, v))


@pytest.mark.parametrize("budget,S,k", [(0.005, 73397, 367), (0.005, 8192, 41), (0.01, 32768, 328),
                                        (0.02, 73397, 1468), (0.005, 70000, 350), (0.0, 5, 0),
                                        (1.0, 77, 77), (0.5, 3, 2), (0.05, 600, 30),
                                        (0.07, 100, 7), (1e-12, 1000, 0), (1e-6, 10**7, 10)])
def test_repair_count(budget, S, k):
    assert oracle.repair_count(budget, S) == k


def test_repair_count_rejects_bad_budget():
    for b in (-0.1, 1.5, math.nan):
        with pytest.raises(ValueError):
            oracle.repair_count(b, 10)


def test_budget_zero_equals_no_repair():
    q, k, v = _head()
    rows = np.arange(0, 2048, 16)
    a = oracle.expcast_attention_head(q, k, v, rows=rows, budget=0.0)["out"]
    ph = oracle.prepare_head(q, k, v, budget=0.0)
    assert ph.repair is None
    b = oracle.expcast_attention_head(q, k, v, rows=rows, ph=ph)["out"]
    assert np.array_equal(a, b)


def _pairwise(xs):
    """pairwise summation by recursive halving"""
    if len(xs) == 1:
        return xs[0]
    h = len(xs) // 2
    return _pairwise(xs[:h]) + _pairwise(xs[h:])


def test_selection_matches_brute_force():
    """Energies recomputed token by token with Python floats (fp32 residual via
    numpy scalars, float64 squares added by recursive halving), then a plain
    sort: the selected set must match exactly."""
    q, k, v = _head(S=600)
    vc, sv = oracle.quantize_head(v)
    rp = oracle.repair_select(v, vc, sv, 0.05)
    dec = oracle.decode(vc)
    energies = []
    for j in range(len(v)):
        sq = []
        for c in range(128):
            r = np.float32(np.float32(v[j, c]) - np.float32(sv) * np.float32(dec[j, c]))
            sq.append(float(r) * float(r))
        energies.append(_pairwise(sq))
    assert np.array_equal(rp.energy, np.array(energies))
    kk = math.ceil(0.05 * 600)
    order = sorted(range(len(v)), key=lambda j: (-energies[j], j))
    assert rp.k == kk
    assert list(rp.sel) == sorted(order[:kk])


def test_ties_take_lower_index():
    v = np.zeros((10, 128))
    v[[2, 5, 7], 0] = 3.0 * 2 ** -12      # equal residual energy (rounds to 0 in E4M3 at this scale)
    v[0, 1] = 1.0                          # sets the head scale
    vc, sv = oracle.quantize_head(v)
    rp = oracle.repair_select(v, vc, sv, 0.2)   # k = 2
    assert list(rp.sel) == [2, 5]


def _v_effective(v, budget):
    vc, sv = oracle.quantize_head(v)
    veff = float(sv) * oracle.decode(vc)
    rp = oracle.repair_select(v, vc, sv, budget)
    if rp.k:
        veff[rp.sel] += float(rp.sr) * oracle.decode(rp.rc)
    return veff, rp


def test_value_error_non_increasing_in_budget_and_hits_outliers():
    _, _, v = _head(S=4096)
    errs = []
    for b in (0.0, 0.005, 0.01, 0.02, 0.1, 1.0):
        veff, rp = _v_effective(v, b)
        errs.append(oracle.rel_l2(veff, v))
    assert all(e1 <= e0 + 1e-12 for e0, e1 in zip(errs, errs[1:])), errs
    assert errs[-1] < 0.002          # full repair leaves only the residual's own E4M3 rounding
    # the outlier tokens (|v| far above the bulk) carry the largest residuals,
    # so nearly all of them are among the first ones repaired
    _, rp = _v_effective(v, 0.01)
    big = np.where(np.abs(v).max(axis=1) > 8.0)[0]
    assert 0 < len(big) <= rp.k
    assert len(set(big) & set(rp.sel)) >= 0.9 * len(big)


def test_repair_output_is_attention_over_repaired_values():
    """With repair, the output equals sum_j P_j (sv dec(v_j) + sr dec(r_j)) / L
    with the unrepaired row sums: the residual changes V, not the weights."""
    q, k, v = _head(S=1024)
    rows = np.arange(0, 1024, 32)
    r = oracle.expcast_attention_head(q, k, v, rows=rows, budget=0.05)
    ph = r["ph"]
    veff = float(ph.sv) * oracle.decode(ph.vc)
    veff[ph.repair.sel] += float(ph.repair.sr) * oracle.decode(ph.repair.rc)
    x = oracle.log2_logits(ph, rows, 1 / math.sqrt(128))
    P = oracle.VALUES[oracle.expcast_codes(x, oracle.bitaligned_row_max(x))]
    want = (P @ veff) / P.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-13)
    r0 = oracle.expcast_attention_head(q, k, v, rows=rows, budget=0.0)
    assert np.array_equal(r["L"], r0["L"]) and np.array_equal(r["M"], r0["M"])
