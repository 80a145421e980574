"""Pins for the oracle's E4M3 codec: the format definition, an independent
arithmetic encoder written here, and torch's float8_e4m3fn cast."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def encode_arith(x):
    """Second, independent route: split |x| into binade and mantissa with
    frexp, round the mantissa to 3 bits with numpy's half-to-even rint, then
    assemble the code. Written from the format, not from oracle/e4m3.py."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.int64)
    nz = a > 0
    _, ex = np.frexp(a[nz])                 # a = f * 2^ex with f in [0.5, 1)
    e = ex - 1                              # a in [2^e, 2^(e+1))
    e = np.maximum(e, -6)                   # below 2^-6 the quantum stays 2^-9
    quantum = np.ldexp(1.0, e - 3)
    n = np.rint(a[nz] / quantum)            # exact division by a power of two
    val = n * quantum
    val = np.minimum(val, 448.0)
    _, ex2 = np.frexp(val)
    e2 = np.maximum(ex2 - 1, -6)
    sub = val < 2.0 ** -6
    m = np.where(sub, val / 2.0 ** -9, val / np.ldexp(1.0, e2) * 8 - 8)
    code = np.where(sub, m, (e2 + 7) * 8 + m)
    out[nz] = code.astype(np.int64)
    out |= np.signbit(x).astype(np.int64) << 7
    return out.astype(np.uint8)


def all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    f32 = bits.view(np.float32)
    return f32[np.isfinite(f32)].astype(np.float64)


def test_format_constants_match_spec():
    g = _golden("e4m3_format.json")
    assert e4m3.VALUES[g["max_finite_code"]] == g["max_finite"]
    assert e4m3.VALUES[8] == g["min_normal"]
    assert e4m3.VALUES[1] == g["min_subnormal"]
    assert e4m3.VALUES[0] == 0.0
    assert np.isnan(e4m3.decode(np.array([g["nan_code"], 0x80 | g["nan_code"]]))).all()
    assert np.all(np.diff(e4m3.VALUES) > 0)
    assert e4m3.decode(np.array([0x38]))[0] == 1.0
    assert e4m3.decode(np.array([0xB8]))[0] == -1.0


def test_log2_relation_on_powers_of_two():
    """The byte of 2^k is exactly 8*k + 56 across the normal range (the
    relation the ExpCast-FP8 section builds on)."""
    g = _golden("e4m3_format.json")
    k0, k1 = g["powers_of_two_k_range"]
    for k in range(k0, k1 + 1):
        c = int(e4m3.encode(np.array([2.0 ** k]))[0])
        assert c == g["log2_relation_slope"] * k + g["log2_relation_offset"]
    # and approximately for every normal value: |code - (8 log2 v + 56)| < 1
    codes = np.arange(8, 127)
    approx = 8 * np.log2(e4m3.VALUES[codes]) + 56
    assert np.abs(codes - approx).max() < 1.0


def test_round_trip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = e4m3.encode(e4m3.decode(codes))
    assert np.array_equal(back, codes)


def test_ties_go_to_even_code_and_saturation():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    # 1.1875 is halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A
    got = e4m3.encode(np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10]))
    assert list(got) == [0x38, 0x3A, 0xB8, 0x00, 0x02]
    got = e4m3.encode(np.array([432.0, 440.0, 448.0, 460.0, 1e9, -1e9]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert e4m3.encode(np.array([416.0]))[0] == 0x7D
    assert e4m3.encode(np.array([-0.0]))[0] == 0x80


def test_encode_matches_arithmetic_route_on_every_bf16():
    x = all_bf16_values()
    assert np.array_equal(e4m3.encode(x), encode_arith(x))


def test_encode_matches_arithmetic_route_random():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200_000) * np.exp2(rng.uniform(-14, 10, 200_000))
    assert np.array_equal(e4m3.encode(x), encode_arith(x))
    # exact midpoints of neighbouring grid values
    mids = 0.5 * (e4m3.VALUES[:-1] + e4m3.VALUES[1:])
    assert np.array_equal(e4m3.encode(mids), encode_arith(mids))


def test_encode_matches_torch_cast_within_range():
    """torch's float8_e4m3fn cast (round to nearest even) agrees wherever it
    does not overflow; torch gives NaN above the grid where we saturate."""
    x = all_bf16_values()
    x = x[np.abs(x) <= 448.0]
    t = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(x), t)
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-12, 8, 100_000))).astype(np.float32)
    y = y[np.abs(y) <= 448.0]
    t = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(y.astype(np.float64)), t)


def test_nan_rejected():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([1.0, math.nan]))
