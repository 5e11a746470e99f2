"""GPU parity of attn_decode against the fp64 decode oracle.

Tolerances: the bf16 attention bar (max-abs <= 2e-2, L1-rel <= 5e-3 over O)
and LSE max-abs <= 2^-8. Each chunk's softmax denominator is the sum of its
bf16-rounded probabilities (each within 2^-9 relative), and the merge adds
fp32 rounding only, so the reasoning of the prefill LSE bound carries over.
"""
import math

import pytest
import torch

from attn_inputs import make_qkv
from oracle import attention_decode, attention_two_pass, max_abs, l1_rel

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 2.0 ** -8


def decode_inputs(B, H, Nq, Nk, d, seed):
    # the queries are the last Nq rows of a length-Nk sequence's Q
    q, k, v = make_qkv(B, H, Nk, d, seed=seed)
    return q[:, :, Nk - Nq:].contiguous(), k, v


def check(o, lse, ref_o, ref_lse, what):
    o, lse = o.double().cpu(), lse.double().cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), what
    ma, l1, la = max_abs(o, ref_o), l1_rel(o, ref_o), max_abs(lse, ref_lse)
    assert ma <= 2e-2 and l1 <= 5e-3 and la <= LSE_MAX_ABS, f"{what}: {ma:.2e} {l1:.2e} {la:.2e}"


@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 1, 1, 1, 64), (2, 3, 1, 1000, 128), (1, 2, 5, 4096, 128),
                                         (2, 2, 32, 300, 64), (1, 1, 17, 17, 128), (1, 4, 8, 20000, 64),
                                         (3, 1, 2, 65, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 3, 64])
def test_decode_vs_oracle(lib, B, H, Nq, Nk, d, causal, splits):
    q, k, v = decode_inputs(B, H, Nq, Nk, d, seed=Nk + Nq + d)
    scale = 1 / math.sqrt(d)
    o, lse = lib.decode(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_decode(q, k, v, scale, causal)
    check(o, lse, ref_o, ref_lse, f"{(B, H, Nq, Nk, d, causal, splits)}")


def test_decode_max_nk(lib):
    """Nk = 2^23 (ATTN_MAX_N), the longest cache the C ABI accepts: the copies'
    offsets and buffer ranges at their limits, and the nontemporal flat copies
    of interior tiles at their largest addresses. Two queries, d = 64, causal,
    the default split count. Inputs from torch's seeded CUDA generator
    (2 Nk d values); oracle in fp64 on the host."""
    Nk, Nq, d = 1 << 23, 2, 64
    g = torch.Generator(device="cuda").manual_seed(97)
    q, k, v = [torch.randn((1, 1, n, d), generator=g, device="cuda").to(torch.bfloat16)
               for n in (Nq, Nk, Nk)]
    o, lse = lib.decode(q, k, v, causal=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_decode(q.cpu(), k.cpu(), v.cpu(), 1 / math.sqrt(d), causal=True)
    check(o, lse, ref_o, ref_lse, "Nk = 2^23")
    del q, k, v, o, lse


@pytest.mark.parametrize("scale", [0.0, -0.4, 1.1])
def test_decode_scales(lib, scale):
    q, k, v = decode_inputs(1, 2, 4, 700, 128, seed=5)
    o, lse = lib.decode(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale, splits=5)
    torch.cuda.synchronize()
    check(o, lse, *attention_decode(q, k, v, scale, True), f"scale={scale}")


def test_decode_matches_the_last_rows_of_prefill(lib):
    B, H, N, d, Nq = 1, 2, 1024, 128, 8
    q, k, v = make_qkv(B, H, N, d, seed=17)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o_full, lse_full = lib.fwd(qd, kd, vd, causal=True)
    o_dec, lse_dec = lib.decode(qd[:, :, N - Nq:].contiguous(), kd, vd, causal=True, splits=4)
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_two_pass(q, k, v, 1 / math.sqrt(d), True, -1)
    check(o_dec, lse_dec, ref_o[:, :, N - Nq:], ref_lse[:, :, N - Nq:], "decode")
    # both kernels within the bar of the oracle, hence of each other
    assert max_abs(o_full[:, :, N - Nq:].cpu(), o_dec.cpu().double()) <= 4e-2


def test_decode_splits_agree_and_reuse_workspace(lib):
    q, k, v = decode_inputs(2, 2, 3, 5000, 128, seed=21)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = torch.empty(lib.load().attn_decode_workspace_bytes(2, 2, 3, 128, 16), dtype=torch.uint8,
                     device="cuda")
    outs = [lib.decode(qd, kd, vd, causal=True, splits=s, workspace=ws) for s in (1, 7, 16)]
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_decode(q, k, v, 1 / math.sqrt(128), True)
    for o, lse in outs:
        check(o, lse, ref_o, ref_lse, "splits")
