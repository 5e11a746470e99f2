"""Pins for the fp64 decode oracle (CPU only): the last rows of the pinned
self-attention oracle, torch's fp64 scaled_dot_product_attention, and brute
force on tiny inputs."""
import math

import pytest
import torch
import torch.nn.functional as F

from oracle import attention_decode, attention_two_pass


def rnd(*shape, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 40), (5, 40), (32, 33), (7, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_is_the_last_rows_of_full_attention(Nq, Nk, causal):
    # the queries are the last Nq positions of a length-Nk sequence
    Q, K, V = rnd(2, 3, Nk, 16, seed=1), rnd(2, 3, Nk, 16, seed=2), rnd(2, 3, Nk, 16, seed=3)
    o, lse = attention_decode(Q[:, :, Nk - Nq:], K, V, 0.3, causal)
    ref_o, ref_lse = attention_two_pass(Q, K, V, 0.3, causal, -1)
    assert torch.allclose(o, ref_o[:, :, Nk - Nq:], atol=1e-12, rtol=0)
    assert torch.allclose(lse, ref_lse[:, :, Nk - Nq:], atol=1e-12, rtol=0)


@pytest.mark.parametrize("Nq,Nk", [(1, 50), (4, 77), (16, 300)])
def test_decode_matches_sdpa(Nq, Nk):
    q, k, v = rnd(1, 2, Nq, 32, seed=4), rnd(1, 2, Nk, 32, seed=5), rnd(1, 2, Nk, 32, seed=6)
    o, lse = attention_decode(q, k, v, 1 / math.sqrt(32), False)
    assert torch.allclose(o, F.scaled_dot_product_attention(q, k, v), atol=1e-12, rtol=0)
    ref_lse = torch.logsumexp((q @ k.transpose(-1, -2)) / math.sqrt(32), dim=-1)
    assert torch.allclose(lse, ref_lse, atol=1e-12, rtol=0)
    # causal with bottom-right alignment through an explicit boolean mask
    allowed = torch.arange(Nk)[None, :] <= (torch.arange(Nq)[:, None] + Nk - Nq)
    oc, _ = attention_decode(q, k, v, 1 / math.sqrt(32), True)
    assert torch.allclose(oc, F.scaled_dot_product_attention(q, k, v, attn_mask=allowed), atol=1e-12, rtol=0)


def test_decode_brute_force():
    q, k, v = rnd(3, 4, seed=7), rnd(6, 4, seed=8), rnd(6, 4, seed=9)
    o, lse = attention_decode(q, k, v, 0.7, True)
    for i in range(3):
        last = 6 - 3 + i
        s = [0.7 * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(4)) for j in range(last + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = math.fsum(w)
        for c in range(4):
            want = math.fsum(w[j] * float(v[j, c]) for j in range(last + 1)) / z
            assert abs(float(o[i, c]) - want) < 1e-13
        assert abs(float(lse[i]) - (mx + math.log(z))) < 1e-13
