"""Error measures between a result and the oracle's output.

TEST INFRASTRUCTURE (see the package docstring).

  max_abs  largest absolute difference over all elements
  l1_rel   sum |o - o*| / sum |o*|   (the "mean relative error" of the bf16
           path, read as a ratio of L1 norms: the mean of per-element ratios
           is undefined where o* is near zero)
  rmse_rel sqrt(mean (o - o*)^2) / sqrt(mean o*^2)   (the fp8 path's error,
           relative to the oracle output's RMS)
"""
from __future__ import annotations

import torch


def _f64(x) -> torch.Tensor:
    if not isinstance(x, torch.Tensor):
        x = torch.as_tensor(x)
    return x.detach().to("cpu", torch.float64)


def max_abs(o, ref) -> float:
    return float((_f64(o) - _f64(ref)).abs().max()) if _f64(ref).numel() else 0.0


def l1_rel(o, ref) -> float:
    r = _f64(ref)
    den = float(r.abs().sum())
    return float((_f64(o) - r).abs().sum()) / den if den > 0 else 0.0


def rmse_rel(o, ref) -> float:
    r = _f64(ref)
    den = float(r.pow(2).mean().sqrt()) if r.numel() else 0.0
    return float((_f64(o) - r).pow(2).mean().sqrt()) / den if den > 0 else 0.0
