"""Pins for the fp64 paged-cache decode oracle (CPU only).

The paged cache is an addressing scheme, so the pins check the addressing
against things that do not share it: brute force with the page arithmetic
written out per position, invariance under any physical page permutation,
the contiguous decode oracle on a cache whose pages are in order, and
independence from whatever the pool holds past a sequence's length.
"""
import math

import pytest
import torch

from oracle import attention_decode, attention_decode_paged, gather_pages


def rnd(*shape, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def paged_problem(B, H, Nq, d, page_size, seq_lens, extra_pages=3, seed=0):
    """Random pool with each sequence's pages scattered over it."""
    max_pages = max((n + page_size - 1) // page_size for n in seq_lens)
    need = sum((n + page_size - 1) // page_size for n in seq_lens)
    P = need + extra_pages
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(P, generator=g)
    table = torch.full((B, max_pages), -1, dtype=torch.int64)
    nxt = 0
    for b, n in enumerate(seq_lens):
        for j in range((n + page_size - 1) // page_size):
            table[b, j] = perm[nxt]
            nxt += 1
    kc, vc = rnd(P, H, page_size, d, seed=seed + 1), rnd(P, H, page_size, d, seed=seed + 2)
    q = rnd(B, H, Nq, d, seed=seed + 3)
    return q, kc, vc, table, torch.tensor(seq_lens)


def test_brute_force_with_the_page_arithmetic_written_out():
    B, H, Nq, d, ps = 2, 2, 3, 4, 2
    q, kc, vc, table, lens = paged_problem(B, H, Nq, d, ps, [5, 3], seed=11)
    scale = 0.7
    o, lse = attention_decode_paged(q, kc, vc, table, lens, scale, causal=True)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            for i in range(Nq):
                pos = n - Nq + i
                w, num = [], [0.0] * d
                for p in range(pos + 1):                      # causal: keys 0..pos
                    page, row = int(table[b, p // ps]), p % ps
                    s = scale * sum(float(q[b, h, i, c]) * float(kc[page, h, row, c]) for c in range(d))
                    w.append((s, page, row))
                mx = max(s for s, _, _ in w)
                den = sum(math.exp(s - mx) for s, _, _ in w)
                for s, page, row in w:
                    for c in range(d):
                        num[c] += math.exp(s - mx) * float(vc[page, h, row, c])
                for c in range(d):
                    assert abs(float(o[b, h, i, c]) - num[c] / den) < 1e-12
                assert abs(float(lse[b, h, i]) - (mx + math.log(den))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_any_physical_page_order_gives_the_same_result(causal):
    q, kc, vc, table, lens = paged_problem(3, 2, 4, 8, 4, [9, 16, 4], seed=21)
    o, lse = attention_decode_paged(q, kc, vc, table, lens, 0.4, causal)
    P = kc.shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5))   # new slot of page p
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    table2 = torch.where(table >= 0, perm[table.clamp(min=0)], table)
    o2, lse2 = attention_decode_paged(q, kc2, vc2, table2, lens, 0.4, causal)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_pages_in_order_are_the_contiguous_cache(causal):
    B, H, Nq, d, ps, n = 2, 3, 5, 16, 8, 40
    K, V = rnd(B, H, n, d, seed=31), rnd(B, H, n, d, seed=32)
    q = rnd(B, H, Nq, d, seed=33)
    npg = n // ps
    # page b * npg + j holds positions j*ps .. of sequence b
    kc = K.reshape(B, H, npg, ps, d).permute(0, 2, 1, 3, 4).reshape(B * npg, H, ps, d)
    vc = V.reshape(B, H, npg, ps, d).permute(0, 2, 1, 3, 4).reshape(B * npg, H, ps, d)
    table = torch.arange(B * npg).reshape(B, npg)
    o, lse = attention_decode_paged(q, kc, vc, table, torch.tensor([n, n]), 0.25, causal)
    ref_o, ref_lse = attention_decode(q, K, V, 0.25, causal)
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)


def test_rows_past_the_sequence_length_are_never_read():
    q, kc, vc, table, lens = paged_problem(2, 1, 2, 8, 8, [11, 3], seed=41)
    o, lse = attention_decode_paged(q, kc, vc, table, lens, 0.5, False)
    kc2, vc2 = kc.clone(), vc.clone()
    for b, n in enumerate([11, 3]):
        last = int(table[b, (n - 1) // 8])
        kc2[last, :, n % 8 or 8:] = float("nan")
        vc2[last, :, n % 8 or 8:] = float("inf")
    unused = sorted(set(range(kc.shape[0])) - set(table[table >= 0].tolist()))
    kc2[unused], vc2[unused] = float("nan"), float("nan")
    o2, lse2 = attention_decode_paged(q, kc2, vc2, table, lens, 0.5, False)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_gather_returns_positions_in_logical_order():
    ps = 4
    kc = torch.arange(5 * 1 * ps * 1, dtype=torch.float64).reshape(5, 1, ps, 1)
    table = torch.tensor([3, 0, 4])
    got = gather_pages(kc, table, 10, ps)[0, :, 0]
    want = torch.cat([kc[3, 0, :, 0], kc[0, 0, :, 0], kc[4, 0, :2, 0]])
    assert torch.equal(got, want)
