"""fp64 attention for a few queries against a longer key/value sequence.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU-baseline leg.

Decoding with a key/value cache ([JJ] section 3): Nq new queries attend to Nk
>= Nq cached keys and values of the same sequence. The queries are the last
Nq positions: query i sits at position Nk - Nq + i, so with causal masking it
may attend keys j <= Nk - Nq + i (the bottom-right alignment, which for
Nq = Nk is the ordinary causal mask). For one (batch, head):

    s_ij  = scale * <q_i, k_j>            j allowed
    o_i   = sum_j softmax_j(s_i) v_j
    lse_i = ln sum_j exp(s_ij)
"""
from __future__ import annotations

import torch

_ROW_CHUNK = 1024


def attention_decode(q, k, v, scale: float, causal: bool = False):
    """q [..., Nq, d], k and v [..., Nk, d] (Nq <= Nk) -> (o, lse) in fp64."""
    q = torch.as_tensor(q).double()
    k = torch.as_tensor(k).double()
    v = torch.as_tensor(v).double()
    Nq, Nk = q.shape[-2], k.shape[-2]
    if Nq > Nk:
        raise ValueError("decode needs Nq <= Nk")
    o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=torch.float64)
    lse = torch.empty(q.shape[:-1], dtype=torch.float64)
    kt = k.transpose(-1, -2)
    for a in range(0, Nq, _ROW_CHUNK):
        b = min(Nq, a + _ROW_CHUNK)
        s = scale * (q[..., a:b, :] @ kt)
        if causal:
            pos = torch.arange(a, b)[:, None] + (Nk - Nq)        # absolute query positions
            s = s.masked_fill(torch.arange(Nk)[None, :] > pos, -torch.inf)
        m = s.max(dim=-1, keepdim=True).values
        p = torch.exp(s - m)
        l = p.sum(dim=-1, keepdim=True)
        o[..., a:b, :] = (p @ v) / l
        lse[..., a:b] = (m + torch.log(l)).squeeze(-1)
    return o, lse
