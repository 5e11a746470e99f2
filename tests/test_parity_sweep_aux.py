"""GPU parity over seeded random sweeps of the decode, paged-decode, merge and
quantiser kernels.

The grid tests (test_decode.py, test_decode_paged.py, test_merge.py and the
quantiser tests in test_parity.py) vary one or two parameters at a time; each
case here draws all of a kernel's parameters together: batch and heads, query
count, ragged cache lengths, head dimension, causal flag, split count, scale,
page size and pool order, number of partials, the quantiser's mode and the
magnitude of the data. Every case is held to the bar of its grid test:
  decode and paged decode: max-abs <= 2e-2, L1-rel <= 5e-3 over O, LSE
    max-abs <= 2^-8 (the reasoning is in test_decode.py);
  merge: |o - o*| <= 2^-8 |o*| + R 2^-22 max|o_r| elementwise and
    |lse - lse*| <= 2^-20 (|lse*| + 1) + R 2^-22, rows with every partial
    empty exactly o = 0, lse = -inf (test_merge.py);
  quantiser, plain and rotated: codes and descales bit for bit.
"""
import math

import numpy as np
import pytest
import torch

from attn_inputs import make_qkv, rotation_signs
from oracle import attention_decode, attention_decode_paged, lse_merge, quantize as o_quantize
from test_decode import check as check_decode
from test_decode_paged import paged_inputs, run as run_paged

pytestmark = pytest.mark.gpu


def _scale(rng, d):
    r = rng.rand()
    if r < 0.5:
        return 1 / math.sqrt(d)
    if r < 0.6:
        return 0.0
    return float(rng.uniform(-1.0, 1.5)) / math.sqrt(d)


def _decode_cases(n=40, seed=3031):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Nq = int(rng.choice([1, 1, 2, 3, 8, 17, 32]))
        Nk = int(rng.choice([Nq, Nq + 1, 63, 64, 65, 200, 1000, 1537, 4096, 6001]))
        Nk = max(Nk, Nq)
        B, H = int(rng.randint(1, 4)), int(rng.randint(1, 4))
        causal = bool(rng.randint(2))
        splits = int(rng.choice([1, 2, 3, 7, 16, 64, 200]))
        out.append((i, B, H, Nq, Nk, d, causal, splits, _scale(rng, d)))
    return out


@pytest.mark.parametrize("i,B,H,Nq,Nk,d,causal,splits,scale", _decode_cases(), ids=lambda v: None)
def test_decode_sweep(lib, i, B, H, Nq, Nk, d, causal, splits, scale):
    what = f"decode case {i}: B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal} splits={splits} scale={scale:.4f}"
    print(what, flush=True)
    q, k, v = make_qkv(B, H, Nk, d, seed=3100 + i)
    q = q[:, :, Nk - Nq:].contiguous()
    o, lse = lib.decode(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, splits=splits)
    torch.cuda.synchronize()
    check_decode(o, lse, *attention_decode(q, k, v, scale, causal), what)


def _paged_cases(n=30, seed=3203):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        page_size = int(rng.choice([32, 64, 128, 256, 1024]))
        Nq = int(rng.choice([1, 1, 2, 5, 16, 32]))
        B = int(rng.randint(1, 5))
        lens = [int(max(Nq, rng.choice([Nq, 31, 32, 33, 100, 700, 2049, 3000]))) for _ in range(B)]
        H = int(rng.randint(1, 4))
        causal = bool(rng.randint(2))
        splits = int(rng.choice([1, 2, 5, 16, 40]))
        out.append((i, B, H, Nq, d, page_size, tuple(lens), causal, splits, _scale(rng, d)))
    return out


@pytest.mark.parametrize("i,B,H,Nq,d,page_size,lens,causal,splits,scale", _paged_cases(),
                         ids=lambda v: None)
def test_paged_decode_sweep(lib, i, B, H, Nq, d, page_size, lens, causal, splits, scale):
    what = (f"paged case {i}: B{B} H{H} Nq{Nq} d{d} page {page_size} lens {list(lens)} "
            f"causal={causal} splits={splits} scale={scale:.4f}")
    print(what, flush=True)
    # the pool holds each sequence's pages in seeded random order, NaN elsewhere
    q, kc, vc, table, sl = paged_inputs(B, H, Nq, d, page_size, list(lens), seed=3300 + i)
    o, lse = run_paged(lib, q, kc, vc, table, sl, causal=causal, scale=scale, splits=splits)
    check_decode(o, lse, *attention_decode_paged(q, kc, vc, table, sl, scale, causal), what)


def _merge_cases(n=30, seed=3407):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 8, 33, 100, 300]))
        B, H = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        N = int(rng.choice([1, 2, 3, 31, 64, 65, 257, 1000]))
        d = int(rng.choice([64, 128, 256]))
        N = max(1, min(N, 4_000_000 // (R * B * H * d)))   # keeps the host oracle quick
        empty = float(rng.choice([0.0, 0.2, 0.9]))
        mag = float(rng.choice([1.0, 30.0, 1e4]))
        out.append((i, R, B, H, N, d, empty, mag))
    return out


@pytest.mark.parametrize("i,R,B,H,N,d,empty,mag", _merge_cases(), ids=lambda v: None)
def test_merge_sweep(lib, i, R, B, H, N, d, empty, mag):
    what = f"merge case {i}: R{R} B{B} H{H} N{N} d{d} empty={empty} lse scale={mag}"
    print(what, flush=True)
    g = torch.Generator().manual_seed(3500 + i)
    o_p = torch.randn(R, B, H, N, d, generator=g, dtype=torch.float32)
    l_p = torch.randn(R, B, H, N, generator=g, dtype=torch.float32) * mag
    l_p[torch.rand(R, B, H, N, generator=g) < empty] = -math.inf
    o, lse = lib.merge(o_p.cuda(), l_p.cuda())
    torch.cuda.synchronize()
    ref_o, ref_lse = lse_merge(o_p, l_p)
    o, lse = o.double().cpu(), lse.double().cpu()
    none = torch.isneginf(ref_lse)
    assert bool(torch.isneginf(lse[none]).all()) and bool((o[none] == 0).all()), what
    ok = ~none
    bound = 2.0 ** -8 * ref_o.abs() + R * 2.0 ** -22 * float(o_p.abs().max())
    assert bool(((o - ref_o).abs()[ok] <= bound[ok]).all()), what
    lb = 2.0 ** -20 * (ref_lse.abs() + 1) + R * 2.0 ** -22
    assert bool(((lse - ref_lse).abs()[ok] <= lb[ok]).all()), what


def _quant_cases(n=40, seed=3607):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        N = int(rng.choice([1, 2, 127, 128, 129, 255, 256, 500, 1025]))
        B, H = int(rng.randint(1, 3)), int(rng.randint(1, 4))
        per_tensor = bool(rng.randint(2))
        rotated = bool(rng.randint(2))
        outliers = bool(rng.randint(2))
        mag = float(rng.choice([1e-3, 1.0, 3.0, 200.0]))
        out.append((i, B, H, N, d, per_tensor, rotated, outliers, mag))
    return out


@pytest.mark.parametrize("i,B,H,N,d,per_tensor,rotated,outliers,mag", _quant_cases(),
                         ids=lambda v: None)
def test_quantize_sweep(lib, i, B, H, N, d, per_tensor, rotated, outliers, mag):
    what = (f"quantise case {i}: B{B} H{H} N{N} d{d} per_tensor={per_tensor} rotated={rotated} "
            f"outliers={outliers} x{mag}")
    print(what, flush=True)
    x, _, _ = make_qkv(B, H, N, d, seed=3700 + i, outliers=outliers)
    x = (x.double() * mag).to(torch.bfloat16)
    s = rotation_signs(3800 + i, d) if rotated else None
    x8, ds = lib.quantize(x.cuda(), per_tensor=per_tensor,
                          rotation_signs=None if s is None else torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    rc, rds = o_quantize(x, per_tensor=per_tensor, rotation_signs=s)
    assert np.array_equal(x8.cpu().numpy(), rc), what
    assert np.array_equal(ds.cpu().numpy(), rds), what
