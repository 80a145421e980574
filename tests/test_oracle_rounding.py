"""Pins for the oracle's remaining rounding helpers, each against something
other than its own formula: the bf16 rounding of the V-Smooth block means
against torch's float32 -> bfloat16 cast, the pairwise residual energy against
math.fsum and the error bound of pairwise summation, and the quantization
scale of tiny blocks against the range of fp32."""
import math

import numpy as np
import pytest
import torch

import oracle


def _finite_f32_patterns(n, seed):
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    # inputs the kernels can meet: finite values whose bf16 rounding stays finite
    return x[np.isfinite(x) & (np.abs(x) < np.float32(3.38e38))]


def test_to_bf16_matches_torch_cast_on_random_bit_patterns():
    x = _finite_f32_patterns(2_000_000, seed=1)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.to_bf16(x)
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))


def test_to_bf16_matches_torch_cast_on_exact_ties():
    """Values halfway between two bf16 neighbours (low 16 bits 0x8000) go to
    the even one, for both parities of the kept part and both signs; one
    below and one above the halfway point go down and up."""
    rng = np.random.default_rng(2)
    hi = rng.integers(0, 0x7F7F, size=100_000, dtype=np.uint32)
    sign = rng.integers(0, 2, size=hi.size, dtype=np.uint32) << 31
    base = (hi << 16) | sign
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        x = (base | np.uint32(low)).view(np.float32)
        x = x[np.isfinite(x)]
        want = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(oracle.to_bf16(x).view(np.uint64), want.view(np.uint64)), hex(low)


def _pairwise_by_halving(xs):
    """Pairwise summation by recursive halving (the textbook definition: the
    sum of a list is the sum of its two halves' sums)."""
    if len(xs) == 1:
        return xs[0]
    h = len(xs) // 2
    return _pairwise_by_halving(xs[:h]) + _pairwise_by_halving(xs[h:])


def _residual_rows(seed, n=400):
    """fp32 residual rows with widely spread magnitudes, so that the order of
    the additions changes the rounded sum."""
    rng = np.random.default_rng(seed)
    mant = rng.normal(size=(n, 128))
    expo = rng.integers(-30, 10, size=(n, 128))
    return (mant * np.exp2(expo)).astype(np.float32)


def test_energy_is_pairwise_sum_by_recursive_halving():
    r = _residual_rows(3)
    e = oracle.residual_energy(r)
    for i in range(len(r)):
        sq = [float(x) * float(x) for x in r[i]]
        assert e[i] == _pairwise_by_halving(sq), i


def test_energy_within_pairwise_error_bound_of_exact_sum():
    """Pairwise summation of n = 128 non-negative terms errs by at most
    gamma_7 = 7u / (1 - 7u) (u = 2^-53) of the sum; math.fsum is the
    correctly rounded sum."""
    r = _residual_rows(4)
    e = oracle.residual_energy(r)
    u = 2.0 ** -53
    gamma = 7 * u / (1 - 7 * u)
    worst = 0.0
    for i in range(len(r)):
        exact = math.fsum(float(x) * float(x) for x in r[i])
        worst = max(worst, abs(e[i] - exact) / exact)
    assert worst <= gamma


def test_energy_order_is_observable():
    """On these rows the channel-order running sum and the pairwise sum round
    differently for some tokens: the energy is the pairwise one."""
    r = _residual_rows(5)
    e = oracle.residual_energy(r)
    seq = np.array([sum(float(x) * float(x) for x in row) for row in r])   # left to right
    differ = e != seq
    assert differ.any()
    # exact squares: tokens whose squares are all equal powers of two sum exactly either way
    p = np.full((2, 128), np.float32(2.0 ** -3))
    assert np.array_equal(oracle.residual_energy(p), np.full(2, 128 * 2.0 ** -6))


def test_permuted_channels_give_near_tied_energies():
    """Tokens whose residuals are channel permutations of one another have
    equal exact energies; pairwise sums of them differ at most in the last
    bits, within the pairwise bound (this is the data the GPU selection test
    uses to check that ties and near-ties are ranked alike)."""
    rng = np.random.default_rng(6)
    base = _residual_rows(7, n=1)[0]
    rows = np.stack([base[rng.permutation(128)] for _ in range(64)])
    e = oracle.residual_energy(rows)
    exact = math.fsum(float(x) * float(x) for x in base)
    assert np.all(np.abs(e - exact) <= 7 * 2.0 ** -53 * exact * 1.0000001)
    assert len(set(e.tolist())) > 1


@pytest.mark.parametrize("amax,unit", [(0.0, True), (2.0 ** -101, True), (np.nextafter(np.float32(2.0 ** -100), 0), True),
                                       (2.0 ** -100, False), (1e-20, False), (3.0e38, False)])
def test_scale_floor(amax, unit):
    """Below 2^-100 a block takes the unit scale (its elements all round to
    code 0); from 2^-100 up both 448/amax and amax/448 are normal fp32 numbers
    and the block's largest element maps onto 448."""
    s, inv = oracle.quant_scale(amax)
    if unit:
        assert s == 1.0 and inv == 1.0
        x = np.array([amax, -amax, amax / 3])
        c = oracle.quantize_with(x, inv)
        assert np.all((c & 0x7F) == 0)
    else:
        f = np.finfo(np.float32)
        assert f.tiny <= s < f.max and f.tiny <= inv < f.max
        top = np.float32(np.float32(amax) * inv)
        assert abs(float(top) - 448.0) <= 448.0 * 2.0 ** -23
