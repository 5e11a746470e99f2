"""Pins for the fp64 merge of partial attention results (CPU only).

The merge is tied to the attention definition itself: attention over a row's
keys split into disjoint subsets, merged, must equal attention over all of
them. Plus the invariants that make a wrong weight, a missing normalisation,
a wrong log base or a mishandled empty partial fail.
"""
import math

import pytest
import torch

from oracle import attention_two_pass, lse_merge


def qkv(N, d, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(N, d, generator=g, dtype=torch.float64) for _ in range(3)]


@pytest.mark.parametrize("R", [1, 2, 3, 7])
@pytest.mark.parametrize("scale", [0.25, 1.7])
def test_merge_of_key_splits_equals_full_attention(R, scale):
    N, d = 37, 16
    q, k, v = qkv(N, d, seed=R)
    g = torch.Generator().manual_seed(100 + R)
    owner = torch.randint(0, R, (N,), generator=g)     # a random, non-contiguous partition
    owner[:R] = torch.arange(R)                          # every part non-empty
    o_parts, lse_parts = [], []
    for r in range(R):
        idx = torch.nonzero(owner == r).flatten()
        o_r, lse_r = attention_two_pass(q[None, None], k[idx][None, None], v[idx][None, None], scale)
        o_parts.append(o_r[0, 0])
        lse_parts.append(lse_r[0, 0])
    o, lse = lse_merge(torch.stack(o_parts), torch.stack(lse_parts))
    ref_o, ref_lse = attention_two_pass(q[None, None], k[None, None], v[None, None], scale)
    assert torch.allclose(o, ref_o[0, 0], atol=1e-12, rtol=0)
    assert torch.allclose(lse, ref_lse[0, 0], atol=1e-12, rtol=0)


def test_single_partial_is_identity():
    g = torch.Generator().manual_seed(1)
    o_p = torch.randn(1, 5, 8, generator=g, dtype=torch.float64)
    l_p = torch.randn(1, 5, generator=g, dtype=torch.float64) * 10
    o, lse = lse_merge(o_p, l_p)
    assert torch.equal(o, o_p[0]) and torch.allclose(lse, l_p[0], atol=1e-15, rtol=0)


def test_empty_partials_weigh_nothing_and_all_empty_gives_zero():
    g = torch.Generator().manual_seed(2)
    o_p = torch.randn(3, 4, 8, generator=g, dtype=torch.float64)
    l_p = torch.randn(3, 4, generator=g, dtype=torch.float64)
    l_p[1, :] = -math.inf
    o_p[1] = 1e300                     # must not leak through a zero weight
    o, lse = lse_merge(o_p, l_p)
    o2, lse2 = lse_merge(o_p[[0, 2]], l_p[[0, 2]])
    assert torch.allclose(o, o2, atol=1e-14, rtol=0) and torch.allclose(lse, lse2, atol=1e-14, rtol=0)
    l_p[:, 2] = -math.inf
    o, lse = lse_merge(o_p, l_p)
    assert torch.all(o[2] == 0) and math.isinf(lse[2]) and lse[2] < 0


def test_permutation_and_shift():
    g = torch.Generator().manual_seed(3)
    o_p = torch.randn(5, 6, 4, generator=g, dtype=torch.float64)
    l_p = torch.randn(5, 6, generator=g, dtype=torch.float64) * 3
    o, lse = lse_merge(o_p, l_p)
    perm = torch.tensor([3, 0, 4, 1, 2])
    o2, lse2 = lse_merge(o_p[perm], l_p[perm])
    assert torch.allclose(o, o2, atol=1e-14) and torch.allclose(lse, lse2, atol=1e-14)
    # a common shift of every partial's lse shifts the merged lse and leaves o alone
    o3, lse3 = lse_merge(o_p, l_p + 700.0)
    assert torch.allclose(o, o3, atol=1e-12) and torch.allclose(lse + 700.0, lse3, atol=1e-10)


def test_two_partials_closed_form():
    # lse = ln(e^a + e^b); o = (e^a o1 + e^b o2) / (e^a + e^b)
    a, b = 0.3, -1.1
    o1 = torch.tensor([[1.0, 2.0]], dtype=torch.float64)
    o2 = torch.tensor([[-3.0, 0.5]], dtype=torch.float64)
    o, lse = lse_merge(torch.stack([o1, o2]), torch.tensor([[a], [b]], dtype=torch.float64))
    ea, eb = math.exp(a), math.exp(b)
    assert abs(float(lse[0]) - math.log(ea + eb)) < 1e-14
    want = (ea * o1 + eb * o2) / (ea + eb)
    assert torch.allclose(o, want, atol=1e-14, rtol=0)
