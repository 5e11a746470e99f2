"""Pins of the error measures every GPU bar is checked with (oracle.metrics).

Each case has a closed-form answer, chosen so that a plausible slip in a
measure fails at least one of them: a signed instead of absolute maximum, a
mean of per-element ratios instead of a ratio of L1 norms, a missing square
root in the RMS numerator or denominator, a sum instead of a mean, a zero
returned for a nonzero error against a zero reference, or broadcasting of
mismatched shapes.
"""
import math

import pytest
import torch

from oracle import max_abs, l1_rel, rmse_rel


def test_max_abs_closed_forms():
    ref = torch.arange(-12, 89, dtype=torch.float64) / 16   # exact binary fractions
    assert max_abs(ref, ref) == 0.0
    assert max_abs(ref + 0.25, ref) == 0.25
    assert max_abs(ref - 0.25, ref) == 0.25                 # the absolute value, not the signed max
    d = torch.zeros(101, dtype=torch.float64)
    d[7], d[50] = 1.0, -5.0                                  # largest error negative
    assert max_abs(ref + d, ref) == 5.0
    spike = ref.clone()
    spike[100] += 2.0 ** -9
    assert max_abs(spike, ref) == 2.0 ** -9


def test_l1_rel_closed_forms():
    ref = torch.tensor([1.0, -2.0, 3.0, -4.0], dtype=torch.float64)
    assert l1_rel(ref, ref) == 0.0
    assert math.isclose(l1_rel(ref * 1.01, ref), 0.01, rel_tol=1e-12)       # scale error
    assert math.isclose(l1_rel(ref + 0.5, ref), 4 * 0.5 / 10.0, rel_tol=1e-12)  # constant offset
    # a ratio of L1 norms, not a mean of per-element ratios (that would be 0.5)
    assert math.isclose(l1_rel(torch.tensor([2.0, 100.0]), torch.tensor([1.0, 100.0])), 1 / 101,
                        rel_tol=1e-12)


def test_rmse_rel_closed_forms():
    ref = torch.full((64,), 3.0, dtype=torch.float64)
    ref[::2] = -3.0                                          # RMS 3, mean 0
    assert rmse_rel(ref, ref) == 0.0
    # constant offset 0.3 against RMS 3: 0.1 (no sqrt in the denominator:
    # 0.3 / 9; none in the numerator: 0.09 / 3; sums instead of means: the same
    # ratio only by accident of equal counts, so a spike case follows)
    assert math.isclose(rmse_rel(ref + 0.3, ref), 0.1, rel_tol=1e-12)
    assert math.isclose(rmse_rel(ref * 0.98, ref), 0.02, rel_tol=1e-12)
    spike = ref.clone()
    spike[5] += 8.0                                          # one error of 8 in 64 elements
    assert math.isclose(rmse_rel(spike, ref), math.sqrt(64 / 64) / 3, rel_tol=1e-12)
    # mean over elements: one error of 8 among 16 elements of RMS 1
    ones = torch.ones(16, dtype=torch.float64)
    e = ones.clone()
    e[0] += 8.0
    assert math.isclose(rmse_rel(e, ones), math.sqrt(64 / 16), rel_tol=1e-12)


def test_zero_reference_and_nan():
    z = torch.zeros(10, dtype=torch.float64)
    assert l1_rel(z, z) == 0.0 and rmse_rel(z, z) == 0.0 and max_abs(z, z) == 0.0
    one = z.clone()
    one[3] = 1e-30
    assert l1_rel(one, z) == math.inf and rmse_rel(one, z) == math.inf
    nan = torch.ones(10, dtype=torch.float64)
    nan[2] = math.nan
    ref = torch.ones(10, dtype=torch.float64)
    for f in (max_abs, l1_rel, rmse_rel):
        assert not (f(nan, ref) <= 1.0)                      # NaN fails every bar


def test_shapes_must_match_and_dtypes_upcast():
    with pytest.raises(ValueError):
        max_abs(torch.zeros(4, 1), torch.zeros(4))
    with pytest.raises(ValueError):
        l1_rel(torch.zeros(3), torch.zeros(1))
    # bf16 inputs are compared in fp64 after an exact upcast
    a = torch.tensor([1.0, 2.0], dtype=torch.bfloat16)
    b = torch.tensor([1.0078125, 2.0], dtype=torch.float64)   # 1 + 2^-7
    assert max_abs(a, b) == 2.0 ** -7
