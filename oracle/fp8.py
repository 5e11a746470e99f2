"""The E4M3 number format and the per-block quantiser, from their definitions.

TEST INFRASTRUCTURE (see the package docstring).

Format: [JJ] section 1.5 gives E4M3 as 1 sign bit, 4 exponent bits and 3
mantissa bits; [WGC] section 3 maps values onto the range whose maximum is 448,
which is the OCP "E4M3FN" variant: exponent bias 7, no infinities, the two codes
S.1111.111 are NaN, exponent field 0 holds subnormals m/8 * 2^-6, and the
largest finite value is 1.75 * 2^8 = 448.

Rounding: round to nearest, ties to the code with an even mantissa, saturating
at +-448 (a finite input never becomes NaN).

Quantiser ([WGC] section 3, "dynamic per-block scaling factor": the page's
formula multiplies max|Q| and max|K| over a single 448, which is read as one
factor amax/448 per tensor block; the product of the Q and K factors then
rescales QK^T). For each block of 128 rows x d of one (batch, head):

    amax    = max |x|                    (exact)
    r       = fp32(448 / amax)           (fp32 division, correctly rounded)
    descale = fp32(amax / 448)
    code    = e4m3(fp32(x * r))          (fp32 product, then RNE to E4M3)
    amax == 0  =>  r = 1, descale = 1 (all codes 0)
    0 < amax < 448 * 2^-126  =>  r = 2^126, descale = 2^-126

The pages say nothing of blocks this small. There amax / 448 would lie below
the smallest normal fp32 and 448 / amax would overflow (to +inf once amax <
448 / FLT_MAX, which turns 0 * r into NaN). The reading taken: the descale
never goes below the smallest normal fp32, 2^-126, and r is its exact
reciprocal. Every |x * r| is then below 448, so nothing saturates, zeros
encode as 0 and code * descale still approximates x (the tiny values keep
fewer significant bits, as E4M3 subnormals). At amax = 448 * 2^-126 exactly
both rules give the same r and descale.

The fp32 steps are those the GPU quantiser takes: where a floating-point
operation decides an integer code, both sides decide it in the same precision.
Per-tensor mode uses one amax over the whole tensor for every block; it is the
naive baseline the per-block scheme is compared against.
"""
from __future__ import annotations

import math

import numpy as np
import torch

E4M3_MAX = 448.0            # [WGC] section 3
E4M3_EXP_BITS = 4           # [JJ] section 1.5
E4M3_MAN_BITS = 3           # [JJ] section 1.5
E4M3_BIAS = 7
QUANT_BLOCK_ROWS = 128
FP32_MIN_NORMAL = 2.0 ** -126
AMAX_MIN_NORMAL = E4M3_MAX * FP32_MIN_NORMAL     # 7 * 2^-120, exact in fp32


def e4m3_decode(code: int) -> float:
    """Value of one 8-bit E4M3FN code (NaN for S.1111.111)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> E4M3_MAN_BITS) & ((1 << E4M3_EXP_BITS) - 1)
    m = code & ((1 << E4M3_MAN_BITS) - 1)
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


def e4m3_decode_table() -> np.ndarray:
    """fp64 values of all 256 codes."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_decode_table()
_POS_VALUES = _TABLE[:0x7F]          # codes 0x00..0x7E: 0 .. 448, strictly increasing


def e4m3_encode(y) -> np.ndarray:
    """Saturating round-to-nearest-even of fp32 values to E4M3FN codes (uint8).

    Nearest of the two neighbouring representable magnitudes; on a tie, the
    code whose mantissa is even. Magnitudes above 448 give 448. NaN gives 0x7F.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64).ravel()
    nan = np.isnan(a)
    a_c = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS_VALUES, a_c, side="left")     # _POS_VALUES[hi] >= a
    hi = np.minimum(hi, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_c - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a_c == _POS_VALUES[hi], hi, code)
    code = code.astype(np.uint8)
    code = np.where(np.signbit(y.ravel()), code | 0x80, code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    return code.reshape(y.shape)


def _to_f32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float32).numpy()
    return np.asarray(x, dtype=np.float32)


def quantize(x, per_tensor: bool = False, block_rows: int = QUANT_BLOCK_ROWS,
             rotation_signs=None):
    """Quantise x [B, H, N, d] to E4M3 codes with per-block descales.

    rotation_signs: d signs; when given, every row is first rotated as the
    incoherent-processing quantiser does (oracle.rotation.rotate_fp32), and
    the codes and descales are those of the rotated tensor.
    Returns (codes uint8 [B, H, N, d], descale float32 [B, H, ceil(N/128)]).
    """
    x = _to_f32(x)
    if rotation_signs is not None:
        from .rotation import rotate_fp32
        x = rotate_fp32(x, rotation_signs)
    B, H, N, d = x.shape
    nb = -(-N // block_rows)
    codes = np.zeros(x.shape, dtype=np.uint8)
    descale = np.zeros((B, H, nb), dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    global_amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    for b in range(B):
        for h in range(H):
            for rb in range(nb):
                blk = x[b, h, rb * block_rows:(rb + 1) * block_rows]
                amax = global_amax if per_tensor else np.float32(np.max(np.abs(blk)))
                if amax == 0:
                    r = np.float32(1.0)
                    ds = np.float32(1.0)
                elif amax < np.float32(AMAX_MIN_NORMAL):
                    r = np.float32(1.0 / FP32_MIN_NORMAL)
                    ds = np.float32(FP32_MIN_NORMAL)
                else:
                    r = np.float32(f448 / amax)
                    ds = np.float32(amax / f448)
                y = (blk * r).astype(np.float32)             # fp32 product
                codes[b, h, rb * block_rows:(rb + 1) * block_rows] = e4m3_encode(y)
                descale[b, h, rb] = ds
    return codes, descale


def dequantize(codes, descale, block_rows: int = QUANT_BLOCK_ROWS) -> np.ndarray:
    """fp64 values code * descale of its block, [B, H, N, d]."""
    codes = np.asarray(codes)
    descale = np.asarray(descale, dtype=np.float64)
    vals = _TABLE[codes]
    N = codes.shape[2]
    row_scale = np.repeat(descale, block_rows, axis=2)[:, :, :N]
    return vals * row_scale[..., None]
