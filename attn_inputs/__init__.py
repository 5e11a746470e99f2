"""Seeded synthetic inputs for the attention forward pass.

Shared by the parity tests, the benchmark and the oracle's callers. This module
holds no attention arithmetic: it only draws random numbers, rounds them to
bf16 and names the five workloads (shape, mask, dtype, scale). The oracle and
the HIP path both take the tensors it returns.

Recipe (the same for every workload):
  * one numpy PCG64 stream per (seed, tensor, batch, head), so that any single
    head can be regenerated on its own without drawing the whole tensor;
  * fp32 standard normal values of shape [N, d] per head;
  * for the outlier workload, 4 of the d channels (one seeded draw, shared by
    Q, K and V and by every head) are multiplied by 10 before rounding;
  * round-to-nearest-even to bf16 (torch's fp32 -> bf16 cast);
  * the random signs of the incoherent-processing rotation of Q and K: one
    seeded draw of d values, -1 or +1 (rotation_signs).

The workloads follow the "sequence length 8192, head dim 128, batch 16"
measurement of page "Warp Group Cluster 优化" (section 性能与适用场景), the
"fixed length 2048, head dim 128" benchmarking step of page "FlashAttention
V3：优化框架吞吐量的关键技术实践" (section 3.1), and the sliding-window mask of
the same page (section 2.1.2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    window: int          # -1: no window
    dtype: str           # "bf16" or "fp8"
    outliers: bool       # 4 of d channels scaled by 10
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def as_dict(self) -> dict:
        out = asdict(self)
        out["scale"] = self.scale
        return out


# The five workloads, smallest first. Seeds are 1000 + index.
WORKLOADS = [
    Workload("noncausal_b1h2n256d64_bf16", 1, 2, 256, 64, False, -1, "bf16", False, 1000),
    Workload("causal_b4h16n2048d128_bf16", 4, 16, 2048, 128, True, -1, "bf16", False, 1001),
    Workload("noncausal_b16h16n8192d128_bf16", 16, 16, 8192, 128, False, -1, "bf16", False, 1002),
    Workload("noncausal_b8h16n8192d128_fp8_outliers", 8, 16, 8192, 128, False, -1, "fp8", True, 1003),
    Workload("causal_window1024_b2h32n16384d64_bf16", 2, 32, 16384, 64, True, 1024, "bf16", False, 1004),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def outlier_channels(seed: int, d: int, count: int = 4) -> np.ndarray:
    """The channel indices scaled by 10 (one draw per seed, shared by Q, K, V)."""
    rng = np.random.default_rng([seed, 99])
    return np.sort(rng.permutation(d)[:count])


def rotation_signs(seed: int, d: int) -> np.ndarray:
    """d random signs (int8, -1 or +1) for the incoherent-processing rotation
    of Q and K: one seeded draw, shared by Q and K and by every head."""
    rng = np.random.default_rng([seed, 77])
    return np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)


def head_fp32(seed: int, tensor: str, b: int, h: int, N: int, d: int,
              outliers: bool = False) -> np.ndarray:
    """fp32 [N, d] draw for one head of one tensor, before bf16 rounding."""
    rng = np.random.default_rng([seed, TENSOR_IDS[tensor], b, h])
    x = rng.standard_normal((N, d), dtype=np.float32)
    if outliers:
        x[:, outlier_channels(seed, d)] *= np.float32(10.0)
    return x


def head_bf16(seed: int, tensor: str, b: int, h: int, N: int, d: int,
              outliers: bool = False) -> torch.Tensor:
    """bf16 [N, d] CPU tensor for one head (RNE rounding of head_fp32)."""
    return torch.from_numpy(head_fp32(seed, tensor, b, h, N, d, outliers)).to(torch.bfloat16)


def make_tensor(seed: int, tensor: str, B: int, H: int, N: int, d: int,
                outliers: bool = False, device: str | torch.device = "cpu") -> torch.Tensor:
    """bf16 [B, H, N, d] tensor built head by head (each head is head_bf16)."""
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        for h in range(H):
            out[b, h].copy_(head_bf16(seed, tensor, b, h, N, d, outliers))
    return out


def make_qkv(B: int, H: int, N: int, d: int, seed: int, outliers: bool = False,
             device: str | torch.device = "cpu"):
    """(q, k, v) bf16 [B, H, N, d] tensors for an arbitrary shape."""
    return tuple(make_tensor(seed, t, B, H, N, d, outliers, device) for t in ("q", "k", "v"))


def workload_qkv(w: Workload, device: str | torch.device = "cpu", B: int | None = None):
    """(q, k, v) for a named workload; B overrides the batch (same per-head draws)."""
    return make_qkv(w.B if B is None else B, w.H, w.N, w.d, w.seed, w.outliers, device)


def workload_head(w: Workload, b: int, h: int):
    """(q, k, v) bf16 [N, d] CPU tensors of one head of a workload."""
    return tuple(head_bf16(w.seed, t, b, h, w.N, w.d, w.outliers) for t in ("q", "k", "v"))
