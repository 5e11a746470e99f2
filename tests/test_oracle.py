"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: torch's fp64
scaled_dot_product_attention (a library routine), brute-force fsum loops on
tiny inputs, closed forms, and invariants of the mathematics. A dropped scale,
a wrong sign, a transposed operand, an off-by-one in the window or a wrong log
base fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (allowed_range, attention_two_pass, attention_online, probabilities,
                    attention_rows)
from attn_inputs import make_qkv

MASKS = [(False, -1), (True, -1), (True, 0), (True, 3), (False, 0), (False, 2), (True, 100), (False, 100)]


def qkv(B, H, N, d, seed=0, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, N, d, generator=g, dtype=dtype) for _ in range(3)]


def dense_band_mask(N, causal, window):
    """Allowed matrix built the way the sliding-window page draws it: row i
    allows keys max(0, i-w) .. i+w ([YT] 2.1.2), then cut at j <= i if causal."""
    m = torch.zeros((N, N), dtype=torch.bool)
    for i in range(N):
        if window >= 0:
            m[i, max(0, i - window):i + window + 1] = True
        else:
            m[i, :] = True
    if causal:
        m &= torch.ones((N, N), dtype=torch.bool).tril()
    return m


def brute(q, k, v, scale, causal, window):
    """Per-element fsum loops, one head."""
    N, d = q.shape
    o = np.zeros((N, v.shape[1]))
    lse = np.full(N, -math.inf)
    for i in range(N):
        lo, hi = allowed_range(i, N, causal, window)
        js = list(range(lo, hi))
        if not js:
            continue
        s = [scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(d)) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(e[t] * float(v[js[t], c]) for t in range(len(js))) / l
        lse[i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("causal,window", MASKS)
def test_brute_force_tiny(causal, window):
    q, k, v = qkv(1, 1, 13, 5, seed=1)
    o, lse = attention_two_pass(q, k, v, 0.37, causal, window)
    ob, lb = brute(q[0, 0], k[0, 0], v[0, 0], 0.37, causal, window)
    assert np.allclose(o[0, 0].numpy(), ob, atol=1e-13, rtol=0)
    assert np.allclose(lse[0, 0].numpy(), lb, atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal,window", MASKS)
def test_sdpa_fp64(causal, window):
    """Library routine: torch's fp64 SDPA with the page's dense band mask."""
    B, H, N, d = 2, 3, 70, 16
    q, k, v = qkv(B, H, N, d, seed=2)
    scale = 1 / math.sqrt(d)
    o, lse = attention_two_pass(q, k, v, scale, causal, window)
    mask = dense_band_mask(N, causal, window)
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    assert (o - ref).abs().max() < 1e-12
    s = torch.where(mask, scale * q @ k.transpose(-1, -2), torch.tensor(-math.inf, dtype=torch.float64))
    assert (lse - torch.logsumexp(s, dim=-1)).abs().max() < 1e-12


def test_sdpa_is_causal_flag():
    q, k, v = qkv(1, 2, 40, 8, seed=3)
    o, _ = attention_two_pass(q, k, v, 0.5, True, -1)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.5)
    assert (o - ref).abs().max() < 1e-12


def test_rows_of_p_sum_to_one():
    q, k, _ = qkv(1, 1, 50, 8, seed=4)
    for causal, window in MASKS:
        p = probabilities(q[0, 0], k[0, 0], 0.3, causal, window)
        assert (p.sum(dim=1) - 1).abs().max() < 1e-12
        assert (p >= 0).all()
        allowed = dense_band_mask(50, causal, window)
        assert (p[~allowed] == 0).all()


def test_output_is_p_times_v():
    q, k, v = qkv(1, 1, 33, 8, seed=5)
    p = probabilities(q[0, 0], k[0, 0], 0.3, True, 7)
    o, _ = attention_two_pass(q, k, v, 0.3, True, 7)
    assert (o[0, 0] - p @ v[0, 0]).abs().max() < 1e-12


@pytest.mark.parametrize("causal,window", MASKS)
def test_constant_v_gives_constant_output(causal, window):
    q, k, _ = qkv(1, 2, 45, 8, seed=6)
    v = torch.full((1, 2, 45, 8), 0.625, dtype=torch.float64)
    o, _ = attention_two_pass(q, k, v, 0.4, causal, window)
    assert (o - 0.625).abs().max() < 1e-13


def test_kv_row_permutation_invariance():
    q, k, v = qkv(2, 2, 64, 16, seed=7)
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(8))
    o1, l1 = attention_two_pass(q, k, v, 0.25)
    o2, l2 = attention_two_pass(q, k[:, :, perm], v[:, :, perm], 0.25)
    assert (o1 - o2).abs().max() < 1e-12 and (l1 - l2).abs().max() < 1e-12


def test_permutation_is_not_invariant_under_causal_mask():
    """Sanity of the previous pin: with a mask the permutation must matter."""
    q, k, v = qkv(1, 1, 32, 8, seed=9)
    perm = torch.arange(31, -1, -1)
    o1, _ = attention_two_pass(q, k, v, 0.25, True)
    o2, _ = attention_two_pass(q, k[:, :, perm], v[:, :, perm], 0.25, True)
    assert (o1 - o2).abs().max() > 1e-3


@pytest.mark.parametrize("tile", [1, 7, 64, 100])
@pytest.mark.parametrize("causal,window", MASKS)
def test_online_equals_two_pass(tile, causal, window):
    q, k, v = qkv(1, 2, 100, 16, seed=10)
    o1, l1 = attention_two_pass(q, k, v, 0.3, causal, window)
    o2, l2 = attention_online(q, k, v, 0.3, causal, window, tile=tile)
    assert (o1 - o2).abs().max() < 1e-12
    assert (l1 - l2).abs().max() < 1e-12


@pytest.mark.parametrize("causal,window", MASKS)
def test_scale_zero_closed_form(causal, window):
    """scale = 0: uniform weights over A(i): o_i = mean of v over A(i), lse_i = ln|A(i)|."""
    N = 37
    q, k, v = qkv(1, 1, N, 8, seed=11)
    o, lse = attention_two_pass(q, k, v, 0.0, causal, window)
    for i in range(N):
        lo, hi = allowed_range(i, N, causal, window)
        assert (o[0, 0, i] - v[0, 0, lo:hi].mean(dim=0)).abs().max() < 1e-13
        assert abs(float(lse[0, 0, i]) - math.log(hi - lo)) < 1e-13


def test_single_key_cases():
    """N = 1, causal row 0 and window 0 reduce to o_i = v_j, lse_i = scale q_i.k_j."""
    q, k, v = qkv(1, 1, 1, 8, seed=12)
    o, lse = attention_two_pass(q, k, v, 0.7)
    assert (o[0, 0, 0] - v[0, 0, 0]).abs().max() < 1e-15
    assert abs(float(lse[0, 0, 0]) - 0.7 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-13
    q, k, v = qkv(1, 1, 20, 8, seed=13)
    o, lse = attention_two_pass(q, k, v, 0.7, True)
    assert (o[0, 0, 0] - v[0, 0, 0]).abs().max() < 1e-15
    for causal in (True, False):
        o, lse = attention_two_pass(q, k, v, 0.7, causal, 0)
        assert (o[0, 0] - v[0, 0]).abs().max() < 1e-15
        assert (lse[0, 0] - 0.7 * (q[0, 0] * k[0, 0]).sum(-1)).abs().max() < 1e-13


def test_large_window_equals_causal():
    q, k, v = qkv(1, 2, 30, 8, seed=14)
    o1, l1 = attention_two_pass(q, k, v, 0.3, True, -1)
    for w in (29, 30, 1000):
        o2, l2 = attention_two_pass(q, k, v, 0.3, True, w)
        assert (o1 - o2).abs().max() == 0 and (l1 - l2).abs().max() == 0
    o3, _ = attention_two_pass(q, k, v, 0.3, True, 28)
    assert (o1 - o3).abs().max() > 0


def test_key_shift_invariance():
    """K <- K + 1 u^T: o unchanged, lse_i shifted by scale * q_i . u (any mask)."""
    q, k, v = qkv(1, 1, 40, 8, seed=15)
    u = torch.randn(8, generator=torch.Generator().manual_seed(16), dtype=torch.float64)
    for causal, window in MASKS:
        o1, l1 = attention_two_pass(q, k, v, 0.3, causal, window)
        o2, l2 = attention_two_pass(q, k + u, v, 0.3, causal, window)
        assert (o1 - o2).abs().max() < 1e-12
        assert (l2 - l1 - 0.3 * (q[0, 0] @ u)).abs().max() < 1e-12


def test_linearity_in_v():
    q, k, v = qkv(1, 1, 40, 8, seed=17)
    _, _, w = qkv(1, 1, 40, 8, seed=18)
    o1, _ = attention_two_pass(q, k, v, 0.3, True, 5)
    o2, _ = attention_two_pass(q, k, w, 0.3, True, 5)
    o3, _ = attention_two_pass(q, k, 2.0 * v - 3.0 * w, 0.3, True, 5)
    assert (o3 - (2.0 * o1 - 3.0 * o2)).abs().max() < 1e-12


def test_causal_and_window_locality():
    N = 40
    q, k, v = qkv(1, 1, N, 8, seed=19)
    i = 17
    o1, _ = attention_two_pass(q, k, v, 0.3, True, 4)
    k2, v2 = k.clone(), v.clone()
    k2[0, 0, i + 1:] += 5.0          # future keys: causal locality
    v2[0, 0, i + 1:] -= 5.0
    k2[0, 0, :i - 4] -= 7.0          # keys older than the window
    v2[0, 0, :i - 4] += 7.0
    o2, _ = attention_two_pass(q, k2, v2, 0.3, True, 4)
    assert (o1[0, 0, i] - o2[0, 0, i]).abs().max() == 0
    k3 = k.clone()
    k3[0, 0, i - 4] += 1.0           # oldest key still inside the window: must matter
    o3, _ = attention_two_pass(q, k3, v, 0.3, True, 4)
    assert (o1[0, 0, i] - o3[0, 0, i]).abs().max() > 0


def test_head_dim_block_split():
    """S_00 = sum over head-dim chunks of Q_0c K_c0 ([JJ] 1.1.1): scores built
    chunk by chunk over d give the same attention (fp64, up to rounding)."""
    q, k, v = qkv(1, 1, 24, 32, seed=20)
    o, lse = attention_two_pass(q, k, v, 0.2, False, -1)
    s = sum(q[0, 0, :, c:c + 8] @ k[0, 0, :, c:c + 8].T for c in range(0, 32, 8)) * 0.2
    p = torch.softmax(s, dim=-1)
    assert (o[0, 0] - p @ v[0, 0]).abs().max() < 1e-12


def test_rows_subset_matches_full():
    q, k, v = qkv(1, 1, 300, 16, seed=21)
    o, lse = attention_two_pass(q, k, v, 0.25, True, 50)
    rows = [0, 1, 49, 50, 51, 199, 299]
    o2, l2 = attention_rows(q[0, 0], k[0, 0], v[0, 0], 0.25, True, 50, rows)
    assert (o[0, 0, rows] - o2).abs().max() == 0 and (lse[0, 0, rows] - l2).abs().max() == 0


def test_empty_allowed_set_convention():
    """A row with no allowed key (only reachable through the row API with a
    causal window cut to nothing) is defined as o = 0, lse = -inf."""
    q, k, v = qkv(1, 1, 4, 4, seed=22)
    # allowed_range with N=4, window 0 is never empty; construct one directly
    assert allowed_range(0, 4, True, 0) == (0, 1)
    assert allowed_range(3, 4, False, 0) == (3, 4)
    lo, hi = allowed_range(2, 0, False, -1)
    assert hi == lo


def test_bf16_inputs_are_exact_upcast():
    q, k, v = make_qkv(1, 1, 16, 8, seed=23)
    o1, _ = attention_two_pass(q, k, v, 0.3)
    o2, _ = attention_two_pass(q.double(), k.double(), v.double(), 0.3)
    assert (o1 - o2).abs().max() == 0
