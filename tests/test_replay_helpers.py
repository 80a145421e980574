"""CPU checks of the GPU tests' decision-replay helpers: bytes computed from
logits moved by less than the allowed bound are accepted (and replayed),
bytes a rounding within the bound cannot produce are rejected."""
import numpy as np
import pytest

import oracle
from gpu_util import validated_codes


@pytest.mark.parametrize("weights", ["expcast", "exp_cast"])
def test_bytes_from_perturbed_logits_are_accepted(weights):
    rng = np.random.default_rng(3)
    x = rng.uniform(-20, 0, size=(64, 500))
    M = np.zeros_like(x)
    codes_of = oracle.expcast_codes if weights == "expcast" else oracle.exp_cast_codes
    delta = 1e-3
    xk = x + rng.uniform(-delta, delta, size=x.shape)
    kc = codes_of(xk, M)
    trace, n = validated_codes(kc, x, M, np.full(x.shape, delta), weights)
    assert n > 0 and n == int((kc != codes_of(x, M)).sum())
    assert np.array_equal(np.where(trace >= 0, trace, codes_of(x, M)), kc)


@pytest.mark.parametrize("weights", ["expcast", "exp_cast"])
def test_bytes_beyond_the_bound_are_rejected(weights):
    rng = np.random.default_rng(4)
    x = rng.uniform(-12, 0, size=(16, 300))
    M = np.zeros_like(x)
    codes_of = oracle.expcast_codes if weights == "expcast" else oracle.exp_cast_codes
    kc = codes_of(x, M).astype(np.int64)
    inner = np.nonzero((kc[0] > 20) & (kc[0] < 110))[0]
    # one code up with a bound far smaller than any entry's distance to a boundary
    mod = kc.copy()
    mod[0, inner[0]] += 1
    with pytest.raises(AssertionError):
        validated_codes(mod, x, M, np.full(x.shape, 1e-9), weights)
    # three codes away with a bound of 0.05 binade (less than one code either side)
    mod = kc.copy()
    mod[0, inner[1]] += 3
    with pytest.raises(AssertionError):
        validated_codes(mod, x, M, np.full(x.shape, 0.05), weights)
    # a bound of two binades admits bytes up to 16 codes away on both paths (8 E4M3 codes per binade)
    mod = kc.copy()
    mod[0, inner[1]] += 3
    trace, n = validated_codes(mod, x, M, np.full(x.shape, 2.0), weights)
    assert n == 1 and trace[0, inner[1]] == kc[0, inner[1]] + 3
