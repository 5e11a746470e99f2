"""GPU parity of attn_decode_paged against the fp64 paged-decode oracle.

Tolerances as for attn_decode (max-abs <= 2e-2, L1-rel <= 5e-3 over O, LSE
max-abs <= 2^-8): the kernel is attn_decode's with different copy addresses.
With the pages in order at d = 128 both kernels run the same tiles in the
same order, so their outputs must agree bit for bit.
"""
import math

import pytest
import torch

from attn_inputs import make_qkv
from oracle import attention_decode_paged, max_abs, l1_rel

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 2.0 ** -8


def paged_inputs(B, H, Nq, d, page_size, seq_lens, seed, spare_pages=5):
    """Seeded queries and a pool holding each sequence's pages in random order;
    unused pool rows hold NaN so that reading one shows in the output."""
    g = torch.Generator().manual_seed(seed)
    pages_per = [(n + page_size - 1) // page_size for n in seq_lens]
    max_pages = max(max(pages_per), 1)
    P = sum(pages_per) + spare_pages
    kc = torch.full((P, H, page_size, d), float("nan"), dtype=torch.bfloat16)
    vc = torch.full((P, H, page_size, d), float("nan"), dtype=torch.bfloat16)
    table = torch.full((B, max_pages), P + 1000, dtype=torch.int32)   # unused entries out of range
    perm = torch.randperm(P, generator=g)
    q = torch.empty((B, H, Nq, d), dtype=torch.bfloat16)
    nxt = 0
    for b, n in enumerate(seq_lens):
        qs, ks, vs = make_qkv(1, H, max(n, Nq), d, seed=seed * 131 + b)
        q[b] = qs[0, :, max(n, Nq) - Nq:]
        for j in range(pages_per[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, j] = page
            r = min(page_size, n - j * page_size)
            kc[page, :, :r] = ks[0, :, j * page_size: j * page_size + r]
            vc[page, :, :r] = vs[0, :, j * page_size: j * page_size + r]
    return q, kc, vc, table, torch.tensor(seq_lens, dtype=torch.int32)


def run(lib, q, kc, vc, table, lens, **kw):
    o, lse = lib.decode_paged(q.cuda(), kc.cuda(), vc.cuda(), table.cuda(), lens.cuda(), **kw)
    torch.cuda.synchronize()
    return o.double().cpu(), lse.double().cpu()


def check(o, lse, ref_o, ref_lse, what):
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), what
    ma, l1, la = max_abs(o, ref_o), l1_rel(o, ref_o), max_abs(lse, ref_lse)
    assert ma <= 2e-2 and l1 <= 5e-3 and la <= LSE_MAX_ABS, f"{what}: {ma:.2e} {l1:.2e} {la:.2e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page_size", [32, 64, 256])
@pytest.mark.parametrize("Nq,seq_lens", [(1, [1, 700, 64, 33]), (4, [4, 1000, 257]),
                                         (32, [32, 95, 2048])])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 3, 16])
def test_paged_decode_vs_oracle(lib, d, page_size, Nq, seq_lens, causal, splits):
    q, kc, vc, table, lens = paged_inputs(len(seq_lens), 2, Nq, d, page_size, seq_lens,
                                          seed=d + page_size + Nq)
    scale = 1 / math.sqrt(d)
    o, lse = run(lib, q, kc, vc, table, lens, causal=causal, scale=scale, splits=splits)
    # the oracle never touches pages or rows a sequence does not own
    ref_o, ref_lse = attention_decode_paged(q, kc, vc, table, lens, scale, causal)
    check(o, lse, ref_o, ref_lse, f"{(d, page_size, Nq, seq_lens, causal, splits)}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.5])
def test_paged_decode_scales(lib, scale):
    q, kc, vc, table, lens = paged_inputs(2, 3, 2, 128, 64, [300, 129], seed=3)
    o, lse = run(lib, q, kc, vc, table, lens, causal=True, scale=scale, splits=4)
    check(o, lse, *attention_decode_paged(q, kc, vc, table, lens, scale, True), f"scale={scale}")


def test_pages_in_order_match_the_contiguous_decode_bit_for_bit(lib):
    B, H, Nq, d, n, ps = 2, 4, 3, 128, 1024, 64
    q, k, v = make_qkv(B, H, n, d, seed=9)
    q = q[:, :, n - Nq:].contiguous()
    npg = n // ps
    kc = k.reshape(B, H, npg, ps, d).permute(0, 2, 1, 3, 4).reshape(B * npg, H, ps, d).contiguous()
    vc = v.reshape(B, H, npg, ps, d).permute(0, 2, 1, 3, 4).reshape(B * npg, H, ps, d).contiguous()
    table = torch.arange(B * npg, dtype=torch.int32).reshape(B, npg)
    lens = torch.full((B,), n, dtype=torch.int32)
    for causal in (False, True):
        o1, l1 = lib.decode(q.cuda(), k.cuda(), v.cuda(), causal=causal, splits=5)
        o2, l2 = lib.decode_paged(q.cuda(), kc.cuda(), vc.cuda(), table.cuda(), lens.cuda(),
                                  causal=causal, splits=5)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_sequence_and_table_entries_outside_the_pool(lib):
    # sequence 1 has no positions (o = 0, lse = -inf); sequence 2's table points
    # outside the pool and past max_pages * page_size: its pages read as zeros
    # (no access outside the pool), and the other sequences are unaffected
    q, kc, vc, table, lens = paged_inputs(3, 2, 1, 128, 32, [200, 1, 64], seed=21)
    lens[1] = 0
    full = int(table[0, 0])            # a page whose 32 rows all hold data
    table[2, :] = torch.tensor([-5, kc.shape[0] + 7] + [full] * (table.shape[1] - 2), dtype=torch.int32)
    lens[2] = 10 ** 6
    o, lse = run(lib, q, kc, vc, table, lens, splits=3)
    ref_o, ref_lse = attention_decode_paged(q[:1], kc, vc, table[:1], lens[:1], 1 / math.sqrt(128))
    check(o[:1], lse[:1], ref_o, ref_lse, "valid sequence")
    assert torch.equal(o[1], torch.zeros_like(o[1])) and torch.isinf(lse[1]).all() and (lse[1] < 0).all()
    assert torch.isfinite(o[2]).all() and torch.isfinite(lse[2]).all()


def test_full_size_sampled(lib):
    # the benchmark's paged decode shape (B32 H32, 16384 positions, 64-position
    # pages in random pool order; 8.6 GB of pool), generated on the device and
    # checked on sampled (b, h)
    B, H, Nq, d, ps, n = 32, 32, 1, 128, 64, 16384
    g = torch.Generator(device="cuda").manual_seed(77)
    P = B * n // ps
    kc = torch.randn((P, H, ps, d), generator=g, device="cuda", dtype=torch.bfloat16)
    vc = torch.randn((P, H, ps, d), generator=g, device="cuda", dtype=torch.bfloat16)
    q = torch.randn((B, H, Nq, d), generator=g, device="cuda", dtype=torch.bfloat16)
    table = torch.randperm(P, generator=g, device="cuda").to(torch.int32).reshape(B, n // ps)
    lens = torch.full((B,), n, dtype=torch.int32, device="cuda")
    o, lse = lib.decode_paged(q, kc, vc, table, lens)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (31, 31), (7, 19)):
        rows = table[b].long()
        ref_o, ref_lse = attention_decode_paged(
            q[b:b + 1, h:h + 1].cpu(), kc[rows, h:h + 1].cpu(), vc[rows, h:h + 1].cpu(),
            torch.arange(n // ps).reshape(1, -1), lens[b:b + 1].cpu(), 1 / math.sqrt(d))
        check(o[b:b + 1, h:h + 1].double().cpu(), lse[b:b + 1, h:h + 1].double().cpu(), ref_o, ref_lse,
              f"sample {(b, h)}")
    del kc, vc
