"""attn_decode_noalloc (the decode entry point that allocates nothing and
keeps its partials in the library's static device buffer) against attn_decode
(the same kernels with a caller's workspace), through the C ABI.

Both entry points run the same kernels on the same inputs with the same split
count, so their outputs must be bit-identical; both must also meet the bf16
bar against the fp64 decode oracle. Two calls in a row, the second smaller
than the first, check that the buffer's leftover contents never reach a
result (every slot a call reads, it has written first), and a call past the
buffer's size is refused without a launch.
"""
import math

import pytest
import torch

from attn_inputs import make_qkv
from oracle import attention_decode, max_abs, l1_rel

pytestmark = pytest.mark.gpu

ATTN_E_SCRATCH = -11


def decode_case(B, H, Nq, Nk, d, seed):
    q, k, v = make_qkv(B, H, Nk, d, seed=seed)
    return q[:, :, Nk - Nq:].contiguous(), k, v


def check_against_decode(lib, B, H, Nq, Nk, d, causal, splits, seed):
    q, k, v = decode_case(B, H, Nq, Nk, d, seed)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = 1 / math.sqrt(d)
    print(f"noalloc case B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal} splits={splits}", flush=True)
    o1, l1 = lib.decode_noalloc(qd, kd, vd, causal=causal, scale=scale, splits=splits)
    o2, l2 = lib.decode(qd, kd, vd, causal=causal, scale=scale, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref_o, ref_lse = attention_decode(q, k, v, scale, causal)
    o1, l1 = o1.double().cpu(), l1.double().cpu()
    assert bool(torch.isfinite(o1).all()) and bool(torch.isfinite(l1).all())
    assert max_abs(o1, ref_o) <= 2e-2 and l1_rel(o1, ref_o) <= 5e-3
    assert max_abs(l1, ref_lse) <= 2.0 ** -8


def test_noalloc_matches_decode_twice_second_smaller(lib):
    # first call: 5 * 2 * 4 * 8 * (4 * 128 + 4) bytes of partials; the second
    # uses fewer splits, fewer rows and d = 64, so it reads a prefix of the
    # buffer the first call filled with other values
    check_against_decode(lib, B=2, H=4, Nq=8, Nk=3000, d=128, causal=True, splits=5, seed=900)
    check_against_decode(lib, B=1, H=2, Nq=3, Nk=500, d=64, causal=False, splits=3, seed=901)


def test_noalloc_largest_call_then_small(lib):
    # the most splits the buffer holds at B4 H8 Nq32 d128 (31 of them), then a
    # one-query call
    check_against_decode(lib, B=4, H=8, Nq=32, Nk=4096, d=128, causal=True, splits=31, seed=902)
    check_against_decode(lib, B=1, H=1, Nq=1, Nk=77, d=128, causal=True, splits=2, seed=903)


def test_noalloc_refuses_a_call_past_the_buffer(lib):
    q, k, v = [t.cuda() for t in decode_case(4, 8, 32, 4096, 128, seed=904)]
    with pytest.raises(lib.AttnError) as e:
        lib.decode_noalloc(q, k, v, causal=True, splits=32)
    assert e.value.code == ATTN_E_SCRATCH
