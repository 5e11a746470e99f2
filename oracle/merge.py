"""fp64 merge of partial attention results over disjoint key sets.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU-baseline leg.

R partial results for the same queries, partial r computed over its own key
set K_r (the sets disjoint, their union the row's allowed set): o_r is the
softmax over K_r applied to V, lse_r = ln sum_{j in K_r} exp(s_ij). Then

    lse = ln sum_r exp(lse_r)
    o   = sum_r exp(lse_r - lse) * o_r

written here with the largest lse_r subtracted first. A partial whose key set
was empty (lse_r = -inf) carries weight 0; if every partial is empty the row
gets o = 0 and lse = -inf, as an empty allowed set does in attention().

This is the output update of the online softmax ([WGC] section 2: each block's
max and sum, the update of the running statistics and the rescale of the
partial output) applied across partial results instead of across key tiles:
the combination a split of the keys over devices or workgroups needs ([WGC]
limitations section on sequence parallelism; [YT] section 2.3.1).
"""
from __future__ import annotations

import torch


def lse_merge(o_parts, lse_parts):
    """o_parts [R, ..., d], lse_parts [R, ...] -> (o [..., d], lse [...]) in fp64."""
    o_parts = torch.as_tensor(o_parts).double()
    lse_parts = torch.as_tensor(lse_parts).double()
    if o_parts.shape[:-1] != lse_parts.shape or o_parts.shape[0] < 1:
        raise ValueError("o_parts must be [R, ..., d] and lse_parts [R, ...] with R >= 1")
    m = lse_parts.max(dim=0).values
    empty = torch.isneginf(m)
    m_safe = torch.where(empty, torch.zeros_like(m), m)
    w = torch.exp(lse_parts - m_safe)            # exp(-inf) = 0 for empty partials
    total = w.sum(dim=0)
    o = (w.unsqueeze(-1) * o_parts).sum(dim=0) / torch.where(empty, torch.ones_like(total), total).unsqueeze(-1)
    o = torch.where(empty.unsqueeze(-1), torch.zeros_like(o), o)
    lse = torch.where(empty, torch.full_like(m, -torch.inf), m_safe + torch.log(total))
    return o, lse
