"""fp64 reference attention: the definition, and the online recurrence.

TEST INFRASTRUCTURE (see the package docstring): imported only by tests, the
smoke check and the benchmark's CPU-baseline leg.

What is computed, for one (batch, head) and query row i, with allowed key set
A(i):

    s_ij   = scale * sum_c q[i, c] * k[j, c]              j in A(i)
    m_i    = max_{j in A(i)} s_ij
    l_i    = sum_{j in A(i)} exp(s_ij - m_i)
    o[i,:] = sum_{j in A(i)} exp(s_ij - m_i) * v[j, :] / l_i
    lse_i  = m_i + ln(l_i)
    A(i) empty  =>  o[i,:] = 0, lse_i = -inf

Sources and readings:
  * The score/softmax/output roles: [WGC] section 1 (QK^T produces S, the
    softmax statistics max and sum, and the second GEMM produces O; the page's
    "S @ V" is read as softmax(S) @ V, since the statistics feed that GEMM).
  * O(N) memory via tiling, S never stored: [WGC] background and section 2.
  * The online recurrence (local max and sum per block, update of the running
    statistics, rescaling of the output): [WGC] section 2; "step-by-step
    accumulation to avoid overflow": [JJ] section 2.4.
  * Mask: [YT] section 2.1.2 builds a 0/1 band where row i allows keys
    max(0, i-w) .. i+w inclusive. Read as a boolean allowed set (an additive
    0 / -inf mask). With causal masking the band is cut at j <= i (N_q = N_k,
    so top-left and bottom-right alignment agree). window = -1 means no band.
  * The per-row log-sum-exp is not on the pages; it is the natural log of the
    softmax denominator over the scaled, masked scores.
"""
from __future__ import annotations

import math

import numpy as np
import torch

_ROW_CHUNK = 2048


def allowed_range(i: int, N: int, causal: bool, window: int) -> tuple[int, int]:
    """Half-open key range [lo, hi) allowed for query row i ([YT] 2.1.2)."""
    lo = max(0, i - window) if window >= 0 else 0
    if causal:
        hi = i + 1
    elif window >= 0:
        hi = min(N, i + window + 1)
    else:
        hi = N
    return lo, max(lo, hi)


def _as_f64(x) -> torch.Tensor:
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(x)
    return x.detach().to(device="cpu", dtype=torch.float64)


def _mask(rows: np.ndarray, cols: np.ndarray, causal: bool, window: int) -> np.ndarray:
    """Boolean allowed[r, c] for absolute row indices `rows` and key indices `cols`."""
    i = rows[:, None]
    j = cols[None, :]
    ok = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        ok &= j <= i
    if window >= 0:
        ok &= j >= i - window
        if not causal:
            ok &= j <= i + window
    return ok


def attention_rows(q, k, v, scale: float, causal: bool = False, window: int = -1,
                   rows=None):
    """Exact two-pass attention for selected query rows of one head.

    q, k, v: [N, d] (any float dtype; upcast exactly to fp64).
    rows: iterable of query indices (default: all).
    Returns (o [len(rows), d] fp64, lse [len(rows)] fp64).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    N = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(list(rows), dtype=np.int64)
    o = torch.zeros((rows.size, v.shape[1]), dtype=torch.float64)
    lse = torch.full((rows.size,), -math.inf, dtype=torch.float64)
    for c0 in range(0, rows.size, _ROW_CHUNK):
        r = rows[c0:c0 + _ROW_CHUNK]
        # key span needed by this chunk (banded when a window is set)
        spans = [allowed_range(int(i), N, causal, window) for i in (r.min(), r.max())]
        lo = min(s[0] for s in spans)
        hi = max(s[1] for s in spans)
        if hi <= lo:
            continue
        cols = np.arange(lo, hi)
        s = scale * (q[torch.from_numpy(r)] @ k[lo:hi].T)           # pass 1: scores
        allowed = torch.from_numpy(_mask(r, cols, causal, window))
        s = s.masked_fill(~allowed, -math.inf)
        m = s.max(dim=1).values                                       # row max
        has = torch.isfinite(m)
        m_safe = torch.where(has, m, torch.zeros_like(m))
        p = torch.exp(s - m_safe[:, None])                            # pass 2: exp, sum
        l = p.sum(dim=1)
        out = (p @ v[lo:hi]) / torch.where(has, l, torch.ones_like(l))[:, None]
        o[c0:c0 + r.size] = torch.where(has[:, None], out, torch.zeros_like(out))
        lse[c0:c0 + r.size] = torch.where(has, m_safe + torch.log(l), lse[c0:c0 + r.size])
    return o, lse


def attention_two_pass(q, k, v, scale: float, causal: bool = False, window: int = -1):
    """Exact attention over [B, H, N, d] tensors.

    Returns (o [B, H, N, d] fp64, lse [B, H, N] fp64).
    """
    q = _as_f64(q)
    B, H, N, d = q.shape
    o = torch.zeros((B, H, N, v.shape[-1]), dtype=torch.float64)
    lse = torch.full((B, H, N), -math.inf, dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_rows(q[b, h], k[b, h], v[b, h], scale, causal, window)
    return o, lse


def attention_online(q, k, v, scale: float, causal: bool = False, window: int = -1,
                     tile: int = 64):
    """Online-softmax attention over [B, H, N, d], key tiles of `tile` rows.

    Follows [WGC] section 2's steps per key block: (1) local max and sum of the
    block, (2) update of the running statistics, (3) rescale of the output
    accumulated so far, then accumulate this block's contribution. All fp64.
    Independent of attention_two_pass (no shared helpers beyond the mask).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    o_all = torch.zeros((B, H, N, dv), dtype=torch.float64)
    lse_all = torch.full((B, H, N), -math.inf, dtype=torch.float64)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            m = torch.full((N,), -math.inf, dtype=torch.float64)    # running max
            l = torch.zeros((N,), dtype=torch.float64)              # running sum
            acc = torch.zeros((N, dv), dtype=torch.float64)         # unnormalised O
            for j0 in range(0, N, tile):
                j1 = min(N, j0 + tile)
                s = scale * (q[b, h] @ k[b, h, j0:j1].T)
                ok = torch.from_numpy(_mask(rows, np.arange(j0, j1), causal, window))
                s = s.masked_fill(~ok, -math.inf)
                m_blk = s.max(dim=1).values                          # (1) local max
                m_new = torch.maximum(m, m_blk)                      # (2) running max
                live = torch.isfinite(m_new)
                ref = torch.where(live, m_new, torch.zeros_like(m_new))
                p = torch.exp(s - ref[:, None])                      # (1) local exp
                alpha = torch.where(live, torch.exp(m - ref), torch.ones_like(m))
                l = alpha * l + p.sum(dim=1)                         # (2) running sum
                acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]      # (3) rescale + add
                m = m_new
            has = l > 0
            o_all[b, h] = torch.where(has[:, None], acc / torch.where(has, l, torch.ones_like(l))[:, None],
                                      torch.zeros_like(acc))
            lse_all[b, h] = torch.where(has, m + torch.log(torch.where(has, l, torch.ones_like(l))),
                                        torch.full_like(m, -math.inf))
    return o_all, lse_all


def probabilities(q, k, scale: float, causal: bool = False, window: int = -1) -> torch.Tensor:
    """The full softmax matrix P [N, N] of one head (small N only)."""
    q = _as_f64(q)
    k = _as_f64(k)
    N = k.shape[0]
    s = scale * (q @ k.T)
    ok = torch.from_numpy(_mask(np.arange(q.shape[0]), np.arange(N), causal, window))
    s = s.masked_fill(~ok, -math.inf)
    m = s.max(dim=1).values
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    e = torch.exp(s - m[:, None])
    tot = e.sum(dim=1, keepdim=True)
    return torch.where(tot > 0, e / torch.where(tot > 0, tot, torch.ones_like(tot)), torch.zeros_like(e))
