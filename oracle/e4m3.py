"""OCP E4M3 (the "FN" variant) codec, written from the format definition.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this.

Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. There are
no infinities; magnitude code 0x7F is NaN, so the largest finite magnitude is
code 0x7E = 448. Exponent field 0 holds the subnormals m * 2^-9.

The VC-Attention write-up (section "ExpCast-FP8") relies on the fact that a
positive E4M3 byte read as an integer is close to 8*log2(v) + 56; with bias 7
that relation is exact for v = 2^k (code 8*(k+7)).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MAX_CODE = 0x7E
NAN_CODE = 0x7F


def _positive_values() -> np.ndarray:
    """float64 value of every non-negative finite magnitude code 0x00..0x7E."""
    vals = np.empty(MAX_CODE + 1, dtype=np.float64)
    for c in range(MAX_CODE + 1):
        e, m = c >> 3, c & 7
        if e == 0:
            vals[c] = m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            vals[c] = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return vals


VALUES = _positive_values()                       # strictly increasing
_MIDPOINTS = 0.5 * (VALUES[:-1] + VALUES[1:])     # exact in float64


def decode(codes) -> np.ndarray:
    """E4M3 byte codes -> float64 values (sign honoured, 0x7F/0xFF -> NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = (c & 0x7F).astype(np.int64)
    out = np.where(mag == NAN_CODE, np.nan, VALUES[np.minimum(mag, MAX_CODE)])
    return np.where((c & 0x80) != 0, -out, out)


def encode(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value; a value exactly halfway
    between two neighbours goes to the one with the even code; magnitudes at or
    above the top of the grid saturate to 448. The sign bit is copied from x
    (so -0.0 and tiny negatives give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("E4M3 encode of NaN")
    a = np.abs(x)
    # i = number of midpoints strictly below a, so MIDPOINTS[i-1] < a <= MIDPOINTS[i]:
    # the nearest grid value is VALUES[i], unless a sits exactly on MIDPOINTS[i].
    i = np.searchsorted(_MIDPOINTS, a, side="left")
    on_mid = (i < len(_MIDPOINTS)) & (a == _MIDPOINTS[np.minimum(i, len(_MIDPOINTS) - 1)])
    code = np.where(on_mid & (i % 2 == 1), i + 1, i)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)
