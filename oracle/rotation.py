"""Incoherent processing: a random-sign Hadamard rotation of Q and K.

TEST INFRASTRUCTURE (see the package docstring).

Page "大模型加速-核心网络算子-Flash Attention V3" (introduction, contribution 3,
and section 3's summary) pairs the FP8 path's block quantisation with
"incoherent processing" (the page's "无相关处理") and gives no further detail.
Reading taken: multiply Q and K by the same random orthogonal matrix
M = diag(s) H / sqrt(d), with H the d x d Sylvester Hadamard matrix and s a
vector of random signs. M M^T = I, so (Q M)(K M)^T = Q K^T and attention is
unchanged, while a few large channels shared by Q and K are spread over all
d channels before the per-block E4M3 quantisation.

Two forms:
  rotate       the definition, (x * s) @ H / sqrt(d) in fp64;
  rotate_fp32  what the GPU quantiser computes, whose fp32 values decide the
               E4M3 codes: y = x * s (exact), the fast Walsh-Hadamard
               butterfly in fp32 with stages h = 1, 2, 4, ..., d/2 (at stage
               h, for every j with bit h clear: y[j], y[j+h] <- y[j] + y[j+h],
               y[j] - y[j+h], each one fp32 rounding), then one fp32 multiply
               by fp32(1/sqrt(d)).
The butterfly's outputs are fixed by its stages alone (each output is one
rounded sum of two values of the previous stage), so any implementation that
keeps this stage order produces the same fp32 values.

The signs are an input, drawn by the seeded input generator (attn_inputs):
entry c counts as -1 where it is negative and +1 otherwise.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), fp64:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def _sign_vector(signs, d: int) -> np.ndarray:
    s = np.asarray(signs).reshape(-1)
    if s.size != d:
        raise ValueError(f"need {d} signs, got {s.size}")
    return np.where(s < 0, -1.0, 1.0)


def _as_f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rotate(x, signs) -> np.ndarray:
    """The definition: (x * s) @ H / sqrt(d) over the last axis, fp64."""
    x = _as_f64(x)
    d = x.shape[-1]
    return (x * _sign_vector(signs, d)) @ hadamard_matrix(d) / math.sqrt(d)


def fwht_fp32(y) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform over the last axis, in fp32,
    stages h = 1, 2, ..., d/2 (see the module docstring)."""
    y = np.array(y, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b          # fp32 + fp32 -> fp32, one rounding
        v[..., 1, :] = a - b
        h *= 2
    return y


def rotate_fp32(x, signs) -> np.ndarray:
    """The rotation as the quantiser computes it in fp32 (see the module
    docstring): signs, butterfly, one multiply by fp32(1 / sqrt(d))."""
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu", torch.float32).numpy()
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    y = x * _sign_vector(signs, d).astype(np.float32)          # exact sign flips
    y = fwht_fp32(y)
    return (y * np.float32(1.0 / math.sqrt(d))).astype(np.float32)
