"""Pins of the incoherent-processing rotation (oracle.rotation) and of the
rotated quantiser (oracle.quantize with rotation_signs), CPU only.

The Hadamard matrix is checked against scipy's (a library construction of the
same Sylvester matrix) and against its defining identity; the fp64 rotation
against the invariances the method relies on (inner products, hence Q K^T and
attention, are unchanged); the fp32 butterfly against the fp64 definition
(exactly on small integers, within its rounding bound otherwise); and the
rotated quantiser against the same round-trip bound as the plain one.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from attn_inputs import rotation_signs, make_qkv
from oracle import (hadamard_matrix, rotate, rotate_fp32, fwht_fp32, quantize, dequantize,
                    attention_two_pass)

DIMS = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_matches_scipy_and_is_orthogonal(d):
    h = hadamard_matrix(d)
    assert np.array_equal(h, scipy.linalg.hadamard(d).astype(np.float64))
    assert np.array_equal(h @ h.T, d * np.eye(d))


def test_hadamard_rejects_non_powers_of_two():
    for d in (0, 3, 96):
        with pytest.raises(ValueError):
            hadamard_matrix(d)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_preserves_inner_products_and_attention(d):
    s = rotation_signs(5, d)
    g = np.random.default_rng(1)
    q = g.standard_normal((40, d))
    k = g.standard_normal((50, d))
    k[:, [3, 17]] *= 10                                      # outlier channels
    rq, rk = rotate(q, s), rotate(k, s)
    assert np.allclose(rq @ rk.T, q @ k.T, rtol=0, atol=1e-11)
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)
    # attention on rotated Q and K equals attention on Q and K
    qt, kt, vt = make_qkv(1, 1, 70, d, seed=3)
    o1, l1 = attention_two_pass(qt, kt, vt, 1 / math.sqrt(d), True, -1)
    o2, l2 = attention_two_pass(torch.from_numpy(rotate(qt, s)), torch.from_numpy(rotate(kt, s)), vt,
                                1 / math.sqrt(d), True, -1)
    assert float((o1 - o2).abs().max()) < 1e-12 and float((l1 - l2).abs().max()) < 1e-12


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_closed_forms(d):
    s = rotation_signs(6, d)
    # a unit vector on channel j becomes s_j times row j of H, over sqrt(d):
    # every output has magnitude 1/sqrt(d) (a single outlier channel is spread
    # evenly over all d channels)
    for j in (0, 5, d - 1):
        e = np.zeros(d)
        e[j] = 1.0
        r = rotate(e, s)
        assert np.allclose(r, s[j] * hadamard_matrix(d)[j] / math.sqrt(d), rtol=0, atol=1e-15)
        assert np.allclose(np.abs(r), 1 / math.sqrt(d), rtol=0, atol=1e-15)
    # the all-plus signs on the first channel's unit vector: the constant vector
    assert np.allclose(rotate(np.eye(d)[0], np.ones(d)), np.full(d, 1 / math.sqrt(d)))
    # H / sqrt(d) is symmetric and orthogonal, so rotating twice with all-plus
    # signs is the identity
    x = np.random.default_rng(2).standard_normal((3, d))
    assert np.allclose(rotate(rotate(x, np.ones(d)), np.ones(d)), x, atol=1e-13)
    # signs: negative entries flip, zero and positive ones do not
    s2 = np.ones(d, dtype=np.int8)
    s2[4] = -7
    s2[9] = 0
    assert np.allclose(rotate(np.eye(d)[4], s2), -hadamard_matrix(d)[4] / math.sqrt(d))
    assert np.allclose(rotate(np.eye(d)[9], s2), hadamard_matrix(d)[9] / math.sqrt(d))


@pytest.mark.parametrize("d", [16, 64, 128])
def test_fwht_fp32_is_exact_on_small_integers(d):
    # sums of integers below 2^12 stay exact in fp32, so the butterfly must
    # equal the matrix product exactly: its pairing and signs are those of
    # Sylvester's H
    x = np.random.default_rng(3).integers(-2000, 2000, size=(20, d)).astype(np.float32)
    assert np.array_equal(fwht_fp32(x).astype(np.float64), x.astype(np.float64) @ hadamard_matrix(d))


@pytest.mark.parametrize("d", [64, 128])
def test_rotate_fp32_within_its_rounding_bound(d):
    # log2(d) butterfly stages and one multiply, each one fp32 rounding of a
    # value no larger than sum |x| (in magnitude): error per element at most
    # (log2(d) + 1) 2^-24 sum|x| / sqrt(d) + 2^-24 |exact|
    s = rotation_signs(7, d)
    g = np.random.default_rng(4)
    x = (g.standard_normal((200, d)) * np.exp(g.uniform(-30, 30, size=(200, 1)))).astype(np.float32)
    x[:, 2] *= 1000
    exact = rotate(x.astype(np.float64), s)
    got = rotate_fp32(x, s).astype(np.float64)
    bound = ((math.log2(d) + 1) * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True)
             / math.sqrt(d) + 2.0 ** -24 * np.abs(exact))
    assert np.all(np.abs(got - exact) <= bound)


@pytest.mark.parametrize("d", [64, 128])
def test_rotated_quantiser_round_trip(d):
    # dequantised codes approximate the rotated tensor within E4M3 rounding,
    # and rotating back recovers x: (y @ H / sqrt(d)) * s inverts the rotation
    s = rotation_signs(8, d)
    x, _, _ = make_qkv(1, 2, 300, d, seed=9, outliers=True)
    codes, ds = quantize(x, rotation_signs=s)
    y = rotate_fp32(x.float().numpy(), s).astype(np.float64)
    deq = dequantize(codes, ds)
    bound = (2.0 ** -4 + 2.0 ** -21) * np.abs(y) + 2.0 ** -10 * np.repeat(ds, 128, axis=2)[:, :, :300, None]
    assert np.all(np.abs(deq - y) <= bound)
    back = (deq @ hadamard_matrix(d) / math.sqrt(d)) * np.where(s < 0, -1.0, 1.0)
    xd = x.double().numpy()
    rms = lambda a: float(np.sqrt(np.mean(a * a)))
    assert rms(back - xd) <= 2.0 ** -4 * rms(xd)
    # plain quantisation is the rotated one with no signs given
    c0, d0 = quantize(x)
    assert not np.array_equal(c0, codes)


def test_fwht_fp32_stage_order_worked_example():
    """The fp32 values depend on the stage order; the quantiser's codes are
    decided from them, so the order h = 1, 2, ..., d/2 is part of the method's
    definition here. Worked by hand for x = [1, 0, e, e], e = 2^-25:
      h = 1: [1 + 0, 1 - 0, e + e, e - e] = [1, 1, 2^-24, 0]   (all exact)
      h = 2: [1 + 2^-24, 1 + 0, 1 - 2^-24, 1 - 0]
             1 + 2^-24 is halfway between 1 and 1 + 2^-23: ties to even, 1;
             1 - 2^-24 is representable (the spacing below 1 is 2^-24).
    so the result is [1, 1, 1 - 2^-24, 1]. (Stages in the other order round
    every 1 +- 2^-25 back to 1 and give [1, 1, 1, 1].)"""
    e = 2.0 ** -25
    y = fwht_fp32(np.array([1.0, 0.0, e, e], dtype=np.float32))
    assert y.tolist() == [1.0, 1.0, 1.0 - 2.0 ** -24, 1.0]
