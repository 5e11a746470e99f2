"""Error measures between a result and the oracle's output.

TEST INFRASTRUCTURE (see the package docstring).

  max_abs  largest absolute difference over all elements
  l1_rel   sum |o - o*| / sum |o*|   (the "mean relative error" of the bf16
           path, read as a ratio of L1 norms: the mean of per-element ratios
           is undefined where o* is near zero)
  rmse_rel sqrt(mean (o - o*)^2) / sqrt(mean o*^2)   (the fp8 path's error,
           relative to the oracle output's RMS)

Both relative measures are 0 for o = o* and +inf for a nonzero error against
an all-zero reference. NaN anywhere in o makes every measure NaN, which fails
every "<=" bar. Shapes must match exactly (no broadcasting).
"""
from __future__ import annotations

import torch


def _f64(x) -> torch.Tensor:
    if not isinstance(x, torch.Tensor):
        x = torch.as_tensor(x)
    return x.detach().to("cpu", torch.float64)


def _pair(o, ref):
    a, r = _f64(o), _f64(ref)
    if a.shape != r.shape:
        raise ValueError(f"shapes differ: {tuple(a.shape)} vs {tuple(r.shape)}")
    return a, r


def _ratio(num: float, den: float) -> float:
    # a nonzero error against an all-zero reference is infinitely large, not 0
    if den > 0:
        return num / den
    return 0.0 if num == 0 else float("inf")


def max_abs(o, ref) -> float:
    a, r = _pair(o, ref)
    return float((a - r).abs().max()) if r.numel() else 0.0


def l1_rel(o, ref) -> float:
    a, r = _pair(o, ref)
    return _ratio(float((a - r).abs().sum()), float(r.abs().sum()))


def rmse_rel(o, ref) -> float:
    a, r = _pair(o, ref)
    if not r.numel():
        return 0.0
    return _ratio(float((a - r).pow(2).mean().sqrt()), float(r.pow(2).mean().sqrt()))
