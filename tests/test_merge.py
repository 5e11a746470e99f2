"""GPU parity of attn_lse_merge against the fp64 merge oracle.

Tolerances: the kernel sums in fp32 and rounds o to bf16 (RNE), so
  |o - o*| <= 2^-8 |o*| + R 2^-22 max_r |o_r|        (bf16 rounding, fp32 sums)
  |lse - lse*| <= 2^-20 (|lse*| + 1) + R 2^-22       (fp32 exp / log / sums)
Rows whose partials are all empty must come out exactly o = 0, lse = -inf.
End to end, partials that are attention over a split of the keys must merge
to full attention within the bf16 attention bar.
"""
import math

import pytest
import torch

from attn_inputs import make_qkv
from oracle import attention_two_pass, lse_merge, max_abs, l1_rel

pytestmark = pytest.mark.gpu


def random_parts(R, B, H, N, d, seed, empty_frac=0.2):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn(R, B, H, N, d, generator=g, dtype=torch.float32)
    l = torch.randn(R, B, H, N, generator=g, dtype=torch.float32) * 3
    drop = torch.rand(R, B, H, N, generator=g) < empty_frac
    l[drop] = -math.inf
    if N > 2:
        l[:, :, :, 1] = -math.inf                  # one row with every partial empty
    return o, l


@pytest.mark.parametrize("R,B,H,N,d", [(1, 1, 1, 1, 64), (2, 1, 2, 129, 128), (5, 2, 1, 300, 256),
                                       (16, 1, 3, 77, 128), (3, 2, 2, 1000, 64), (64, 1, 1, 33, 128)])
def test_merge_vs_oracle(lib, R, B, H, N, d):
    o_p, l_p = random_parts(R, B, H, N, d, seed=R * 100 + N)
    o, lse = lib.merge(o_p.cuda(), l_p.cuda())
    torch.cuda.synchronize()
    ref_o, ref_lse = lse_merge(o_p, l_p)
    o, lse = o.double().cpu(), lse.double().cpu()
    empty = torch.isneginf(ref_lse)
    assert bool(torch.isneginf(lse[empty]).all()) and bool((o[empty] == 0).all())
    ok = ~empty
    bound = 2.0 ** -8 * ref_o.abs() + R * 2.0 ** -22 * float(o_p.abs().max())
    assert bool(((o - ref_o).abs()[ok] <= bound[ok]).all()), float(((o - ref_o).abs() - bound)[ok].max())
    lb = 2.0 ** -20 * (ref_lse.abs() + 1) + R * 2.0 ** -22
    assert bool(((lse - ref_lse).abs()[ok] <= lb[ok]).all())


@pytest.mark.parametrize("R,causal", [(2, False), (4, False), (3, True)])
def test_merge_of_attention_over_key_splits(lib, R, causal):
    """Partial attention over contiguous key blocks (fp64 oracle, stored in
    fp32 as a split-key kernel would write it), merged on the GPU, against
    attention over all keys."""
    B, H, N, d = 1, 2, 256, 128
    q, k, v = make_qkv(B, H, N, d, seed=90 + R)
    scale = 1 / math.sqrt(d)
    bounds = [round(N * r / R) for r in range(R + 1)]
    o_p = torch.empty(R, B, H, N, d, dtype=torch.float32)
    l_p = torch.empty(R, B, H, N, dtype=torch.float32)
    qd = q.double()
    for r in range(R):
        a, b = bounds[r], bounds[r + 1]
        kd, vd = k[:, :, a:b].double(), v[:, :, a:b].double()
        s = scale * qd @ kd.transpose(-1, -2)
        if causal:
            keys = torch.arange(a, b)[None, :]
            rows = torch.arange(N)[:, None]
            s = s.masked_fill(keys > rows, -math.inf)
        lse_r = torch.logsumexp(s, dim=-1)
        p = torch.exp(s - torch.where(torch.isneginf(lse_r), torch.zeros_like(lse_r), lse_r)[..., None])
        o_p[r] = (p @ vd).float()
        l_p[r] = lse_r.float()
    o, lse = lib.merge(o_p.cuda(), l_p.cuda())
    torch.cuda.synchronize()
    ref_o, ref_lse = attention_two_pass(q, k, v, scale, causal, -1)
    assert max_abs(o.cpu(), ref_o) <= 2e-2 and l1_rel(o.cpu(), ref_o) <= 5e-3
    assert max_abs(lse.cpu(), ref_lse) <= 1e-5


def test_merge_caller_outputs_and_stream(lib):
    o_p, l_p = random_parts(3, 1, 2, 50, 128, seed=7, empty_frac=0.0)
    o_p, l_p = o_p.cuda(), l_p.cuda()
    out = torch.full((1, 2, 50, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 2, 50), float("nan"), device="cuda")
    torch.cuda.synchronize()                 # inputs written on the default stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lib.merge(o_p, l_p, out=out, lse=lse, stream=s)
    s.synchronize()
    ref_o, ref_lse = lse_merge(o_p.cpu(), l_p.cpu())
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse[:, :, 2:]).all()
    o2, lse2 = lib.merge(o_p, l_p)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, lse2)       # deterministic
