"""GPU parity over a seeded random sweep of mixed parameters.

The grid tests in test_parity.py vary one or two parameters at a time; here
each case draws dtype (bf16, E4M3 Q/K/V, PV mode), head dimension, ragged
sequence length, batch and heads, causal flag, window, scale and the
quantiser mode together, so that combinations no grid lists are exercised.
Every case is held to the same bar as its grid test (the bf16 bar, or the
elementwise bound against the oracle on the dequantised inputs)."""
import math

import numpy as np
import pytest
import torch

from attn_inputs import make_qkv
from oracle import attention_two_pass
from test_parity import check_bf16, fp8_run, check_fp8_vs_dequantised, fp8pv_run, check_fp8pv

pytestmark = pytest.mark.gpu


def _cases(n=150, seed=2024):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        kind = ["bf16", "fp8", "fp8pv"][i % 3]
        d = int(rng.choice([64, 128, 256] if kind == "bf16" else [64, 128]))
        N = int(rng.choice([1, 2, 31, 64, 65, 127, 129, 255, 257, 511, 700, 1023, 1025, 1600, 2100]))
        B, H = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        causal = bool(rng.randint(2))
        window = -1 if rng.rand() < 0.4 else int(rng.randint(0, N + 64))
        scale = 1 / math.sqrt(d) if rng.rand() < 0.5 else float(rng.uniform(-1.0, 1.5)) / math.sqrt(d)
        per_tensor = bool(rng.randint(2))
        out.append((i, kind, B, H, N, d, causal, window, scale, per_tensor))
    return out


@pytest.mark.parametrize("i,kind,B,H,N,d,causal,window,scale,per_tensor", _cases(),
                         ids=lambda v: None)
def test_random_sweep(lib, i, kind, B, H, N, d, causal, window, scale, per_tensor):
    what = f"case {i}: {kind} B{B} H{H} N{N} d{d} causal={causal} window={window} scale={scale:.4f}"
    print(what, flush=True)
    q, k, v = make_qkv(B, H, N, d, seed=900 + i)
    if kind == "bf16":
        o, lse = lib.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, window=window, scale=scale)
        torch.cuda.synchronize()
        ref_o, ref_lse = attention_two_pass(q, k, v, scale, causal, window)
        check_bf16(o, lse, ref_o, ref_lse, what)
    elif kind == "fp8":
        o, lse, codes = fp8_run(lib, q, k, v, per_tensor, causal, window, scale)
        check_fp8_vs_dequantised(o, lse, codes, scale, causal, window, what, False)
    else:
        o, lse, v8, dv = fp8pv_run(lib, q, k, v, causal, window, scale)
        check_fp8pv(o, lse, q, k, v8, dv, scale, causal, window, what)
