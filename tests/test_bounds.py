"""Reads past the end of a head stay inside the buffer range check.

Every kernel copies K and V tiles through buffer descriptors whose range
check turns a read at or past the head's end into zeros. These tests place
q, k and v at the start of larger buffers whose remainder holds NaN (bf16
0x7FC0, E4M3 0x7F), with ragged lengths, so that the last head's final tile
and the unused tile the pipeline prefetches past it both reach into the NaN
region. If any of those rows were read from memory, P = 0 times V = NaN would
make O NaN. The NaN region is part of the allocation, so these tests cannot
fault, whatever the kernels do. The outputs must be finite and meet the same
bars against the fp64 oracle as the other parity tests.

The caller-supplied output checks of the binding launch nothing: a wrong
device, shape, dtype or layout raises ValueError before any kernel runs.
"""
import math

import numpy as np
import pytest
import torch

from attn_inputs import make_qkv
from oracle import attention_two_pass, attention_decode, max_abs, l1_rel
from test_parity import check_bf16, check_fp8_vs_dequantised, check_fp8pv

pytestmark = pytest.mark.gpu

PAD_BYTES = 1 << 20   # NaN bytes after each tensor: more than any tile the kernels copy


def nan_tailed(t: torch.Tensor) -> torch.Tensor:
    """A copy of t on the GPU, at the start of a buffer whose remaining
    PAD_BYTES hold NaN in t's format."""
    t = t.contiguous()
    n = t.numel()
    pad = PAD_BYTES // t.element_size()
    if t.dtype == torch.bfloat16:
        buf = torch.full((n + pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    else:   # E4M3 codes as bytes; 0x7F is NaN
        buf = torch.full((n + pad,), 0x7F, dtype=torch.uint8, device="cuda")
    view = buf[:n].view(t.shape)
    view.copy_(t.to("cuda").view(view.dtype))
    return view


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 130, 64), (1, 1, 130, 128), (1, 1, 100, 256),
                                     (2, 3, 333, 128), (1, 2, 65, 64), (1, 1, 1, 128)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (False, 40)])
def test_bf16_nan_past_end(lib, B, H, N, d, causal, window):
    q, k, v = make_qkv(B, H, N, d, seed=700 + N + d)
    scale = 1 / math.sqrt(d)
    o, lse = lib.fwd(nan_tailed(q), nan_tailed(k), nan_tailed(v), causal=causal, window=window,
                     scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_two_pass(q, k, v, scale, causal, window)
    check_bf16(o, lse, ref_o, ref_lse, f"nan tail {(B, H, N, d, causal, window)}")


def test_bf16_nan_past_end_wide_grid(lib):
    # B32 H32 N130: 1024 tiles of 256 queries, so d = 128 without a mask runs
    # the 8-wave workgroups; the last head's tail is NaN
    B, H, N, d = 32, 32, 130, 128
    q, k, v = make_qkv(B, H, N, d, seed=711)
    o, lse = lib.fwd(nan_tailed(q), nan_tailed(k), nan_tailed(v))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    for b, h in ((31, 31), (0, 0), (17, 5)):
        sl = lambda t: t[b:b + 1, h:h + 1]
        ref_o, ref_lse = attention_two_pass(sl(q), sl(k), sl(v), 1 / math.sqrt(d), False, -1)
        check_bf16(sl(o), sl(lse), ref_o, ref_lse, f"wide nan tail head {(b, h)}")


@pytest.mark.parametrize("N,d", [(1000, 128), (130, 128)])
def test_bf16_nan_past_end_causal_pairs(lib, N, d):
    # causal with at most 32 query tiles per head: the tile-pair instance
    q, k, v = make_qkv(1, 2, N, d, seed=720 + N)
    o, lse = lib.fwd(nan_tailed(q), nan_tailed(k), nan_tailed(v), causal=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_two_pass(q, k, v, 1 / math.sqrt(d), True, -1)
    check_bf16(o, lse, ref_o, ref_lse, f"paired nan tail N={N}")


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 130, 64), (1, 1, 200, 128), (1, 2, 333, 128),
                                     (1, 1, 1, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_nan_past_end(lib, B, H, N, d, causal):
    q, k, v = make_qkv(B, H, N, d, seed=730 + N + d)
    scale = 1 / math.sqrt(d)
    (q8, dq), (k8, dk), (v8, dv) = [lib.quantize(t.cuda()) for t in (q, k, v)]
    o, lse = lib.fwd(nan_tailed(q8), nan_tailed(k8), nan_tailed(v8), descales=(dq, dk, dv),
                     causal=causal, scale=scale)
    torch.cuda.synchronize()
    codes = [t.cpu().numpy() for t in (q8, dq, k8, dk, v8, dv)]
    check_fp8_vs_dequantised(o.cpu(), lse.cpu(), codes, scale, causal, -1,
                             f"fp8 nan tail {(B, H, N, d, causal)}", False)


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 130, 64), (1, 2, 200, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8pv_nan_past_end(lib, B, H, N, d, causal):
    q, k, v = make_qkv(B, H, N, d, seed=740 + N + d)
    scale = 1 / math.sqrt(d)
    v8, dv = lib.quantize(v.cuda())
    o, lse = lib.fwd(nan_tailed(q), nan_tailed(k), nan_tailed(v8), descales=(None, None, dv),
                     causal=causal, scale=scale)
    torch.cuda.synchronize()
    check_fp8pv(o.cpu(), lse.cpu(), q, k, v8.cpu().numpy(), dv.cpu().numpy(), scale, causal, -1,
                f"fp8 PV nan tail {(B, H, N, d, causal)}")


@pytest.mark.parametrize("Nk,d,splits", [(100, 128, 1), (1000, 128, 3), (70, 64, 1), (1000, 64, 3)])
def test_decode_nan_past_end(lib, Nk, d, splits):
    B, H, Nq = 1, 2, 3
    q, k, v = make_qkv(B, H, Nk, d, seed=750 + Nk + d)
    q = q[:, :, Nk - Nq:].contiguous()
    scale = 1 / math.sqrt(d)
    o, lse = lib.decode(q.cuda(), nan_tailed(k), nan_tailed(v), causal=True, scale=scale,
                        splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_decode(q, k, v, scale, True)
    o, lse = o.double().cpu(), lse.double().cpu()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert max_abs(o, ref_o) <= 2e-2 and l1_rel(o, ref_o) <= 5e-3 and max_abs(lse, ref_lse) <= 2.0 ** -8


# ---- caller-supplied tensors are validated before any launch

def test_fwd_rejects_bad_outputs(lib):
    B, H, N, d = 1, 2, 130, 64
    q, k, v = [t.cuda() for t in make_qkv(B, H, N, d, seed=760)]
    good_o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    good_l = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    bad_outs = [torch.empty((B, H, N, d), dtype=torch.bfloat16),                  # host memory
                torch.empty((B, H, N - 1, d), dtype=torch.bfloat16, device="cuda"),  # short
                torch.empty((B, H, N, d), dtype=torch.float32, device="cuda"),    # dtype
                torch.empty((B, H, d, N), dtype=torch.bfloat16, device="cuda").transpose(2, 3)]
    for bad in bad_outs:
        with pytest.raises(ValueError):
            lib.fwd(q, k, v, out=bad, lse=good_l)
    bad_lses = [torch.empty((B, H, N)), torch.empty((B, H, N - 1), device="cuda"),
                torch.empty((B, H, N), dtype=torch.float64, device="cuda")]
    for bad in bad_lses:
        with pytest.raises(ValueError):
            lib.fwd(q, k, v, out=good_o, lse=bad)


def test_fwd_rejects_bad_descales(lib):
    B, H, N, d = 1, 2, 300, 128
    q, k, v = [t.cuda() for t in make_qkv(B, H, N, d, seed=761)]
    (q8, dq), (k8, dk), (v8, dv) = [lib.quantize(t) for t in (q, k, v)]
    short = dq[:, :, :2].contiguous()
    host = dk.cpu()
    f64 = dv.double()
    for ds in ((short, dk, dv), (dq, host, dv), (dq, dk, f64)):
        with pytest.raises(ValueError):
            lib.fwd(q8, k8, v8, descales=ds)
    with pytest.raises(ValueError):
        lib.fwd(q, k, v8, descales=(None, None, short))


def test_quantize_merge_decode_reject_bad_outputs(lib):
    x = make_qkv(1, 1, 200, 64, seed=762)[0].cuda()
    with pytest.raises(ValueError):
        lib.quantize(x, out=torch.empty((1, 1, 200, 64), dtype=torch.uint8))
    with pytest.raises(ValueError):
        lib.quantize(x, descale=torch.empty((1, 1, 1), device="cuda"))
    op = torch.zeros((2, 1, 1, 8, 64), device="cuda")
    lp = torch.zeros((2, 1, 1, 8), device="cuda")
    with pytest.raises(ValueError):
        lib.merge(op, lp, out=torch.empty((1, 1, 8, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        lib.merge(op, lp, lse=torch.empty((1, 1, 7), device="cuda"))
    q, k, v = [t.cuda() for t in make_qkv(1, 1, 100, 64, seed=763)]
    with pytest.raises(ValueError):
        lib.decode(q[:, :, :2].contiguous(), k, v, out=torch.empty((1, 1, 2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        lib.decode(q[:, :, :2].contiguous(), k, v, workspace=torch.empty(1 << 16, dtype=torch.uint8))
