"""Pins for the oracle's E4M3 model and quantiser (CPU only).

The decode table is checked against torch's float8_e4m3fn type (a library
implementation of the same OCP format) and against the facts the pages print
(4 exponent / 3 mantissa bits, maximum 448); the encoder against torch's
fp32 -> float8_e4m3fn cast over every bf16 bit pattern in range and over
random and tie-constructed fp32 values; the quantiser against a torch-only
re-derivation and against its defining invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (E4M3_MAX, e4m3_decode_table, e4m3_encode, quantize, dequantize,
                    QUANT_BLOCK_ROWS)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_codes(y_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = e4m3_decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], tab[ok])


def test_decode_table_matches_page_facts():
    with open(os.path.join(GOLDEN, "e4m3_facts.json")) as f:
        facts = json.load(f)
    tab = e4m3_decode_table()
    finite = tab[~np.isnan(tab)]
    assert finite.max() == facts["max_finite"] == E4M3_MAX
    assert finite.min() == -facts["max_finite"]
    # 4 exponent bits and 3 mantissa bits: 8 mantissa steps per binade, 16 binades
    assert np.sum(np.isnan(tab)) == facts["nan_codes"]
    pos = np.sort(finite[finite > 0])
    assert pos.size == 2 ** (facts["exponent_bits"] + facts["mantissa_bits"]) - 2
    assert np.isinf(tab).sum() == 0
    assert pos[0] == 2.0 ** facts["min_subnormal_log2"]


def test_encode_all_bf16_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    ok = np.isfinite(y) & (np.abs(y) <= E4M3_MAX)
    y = y[ok]
    assert np.array_equal(e4m3_encode(y), torch_codes(y))


def test_encode_random_fp32_match_torch():
    rng = np.random.default_rng(5)
    parts = [rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 0.02, 1, 30, 150)]
    y = np.concatenate(parts)
    y = y[np.abs(y) <= E4M3_MAX]
    assert np.array_equal(e4m3_encode(y), torch_codes(y))


def test_encode_exact_ties_round_to_even():
    tab = e4m3_decode_table()
    pos = tab[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)     # exact in fp32
    codes = e4m3_encode(mids)
    assert np.all(codes % 2 == 0)
    assert np.array_equal(codes, torch_codes(mids))
    assert np.array_equal(e4m3_encode(-mids), codes | 0x80)


def test_encode_roundtrip_and_saturation():
    tab = e4m3_decode_table()
    fin = np.arange(256)[~np.isnan(tab)]
    vals = tab[fin].astype(np.float32)
    back = e4m3_encode(vals)
    # +0 and -0 both decode to 0; everything else round-trips to its own code
    assert np.array_equal(tab[back], tab[fin])
    sat = e4m3_encode(np.array([449.0, 463.9, 464.0, 1e9, -1e9, -470.0], dtype=np.float32))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def _blocks(x, per_tensor):
    B, H, N, d = x.shape
    nb = -(-N // QUANT_BLOCK_ROWS)
    for b in range(B):
        for h in range(H):
            for rb in range(nb):
                yield b, h, rb, x[b, h, rb * QUANT_BLOCK_ROWS:(rb + 1) * QUANT_BLOCK_ROWS]


@pytest.mark.parametrize("per_tensor", [False, True])
def test_quantize_matches_torch_rederivation(per_tensor):
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(2, 3, 300, 16, generator=g) * torch.rand(2, 3, 300, 1, generator=g) * 20).to(torch.bfloat16)
    codes, ds = quantize(x, per_tensor=per_tensor)
    xf = x.float()
    gmax = xf.abs().max()
    for b, h, rb, blk in _blocks(xf, per_tensor):
        amax = gmax if per_tensor else blk.abs().max()
        r = torch.tensor(448.0, dtype=torch.float32) / amax
        ref = (blk * r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = codes[b, h, rb * 128:(rb + 1) * 128]
        assert np.array_equal(got, ref)
        assert ds[b, h, rb] == np.float32((amax / torch.tensor(448.0)).item())


def test_quantize_invariants():
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(1, 2, 261, 8, generator=g) * 3).to(torch.bfloat16)
    x[0, 1, 128:256] = 0                                    # an all-zero block
    codes, ds = quantize(x)
    assert ds.shape == (1, 2, 3)
    assert np.all(codes[0, 1, 128:256] == 0) and ds[0, 1, 1] == 1.0
    tab = e4m3_decode_table()
    xf = x.double().numpy()
    deq = dequantize(codes, ds)
    for b, h, rb, blk in _blocks(x.float(), False):
        if ds[b, h, rb] == 1.0 and float(blk.abs().max()) == 0:
            continue
        c = codes[b, h, rb * 128:(rb + 1) * 128]
        assert np.abs(tab[c]).max() == 448.0                 # block max lands on 448
        amax = float(blk.abs().max())
        assert abs(448.0 * float(ds[b, h, rb]) - amax) <= amax * 2 ** -23
    # relative error of E4M3 (3 mantissa bits) is at most 2^-4 in the normal range
    normal = np.abs(xf) >= 2.0 ** -6 * np.repeat(ds, 128, axis=2)[:, :, :261, None]
    rel = np.abs(deq - xf)[normal] / np.abs(xf)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-9


def test_per_tensor_descales_are_uniform():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(2, 2, 256, 8, generator=g).to(torch.bfloat16)
    _, ds = quantize(x, per_tensor=True)
    assert np.all(ds == ds.flat[0])
    assert ds.flat[0] == np.float32(float(x.float().abs().max()) / 448.0)


# ---- blocks at every magnitude, including those whose amax / 448 would not
# be a normal fp32 (the quantiser's reading for 0 < amax < 448 * 2^-126)

MAGNITUDES = [2.0 ** -133, 1e-39, 1e-37, 3e-36, 5.2e-36, 7 * 2.0 ** -120, 5.3e-36, 1e-20, 1e-3, 1.0,
              300.0, 1e30, 3.0e38]


def _block_of(amax, n=128, d=16, seed=0):
    """A 128 x d block of values in [-amax, amax] (bf16), its largest magnitude
    amax itself (when amax is a bf16 value), with a few exact zeros."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.rand(n, d, generator=g, dtype=torch.float64) * 2 - 1) * amax
    x[0, 0] = amax
    x[3, :4] = 0.0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("amax", MAGNITUDES)
def test_quantize_round_trip_bound_at_every_magnitude(amax):
    """code * descale reproduces x within E4M3's rounding at any block scale:
    |deq - x| <= (2^-4 + 2^-21) |x| + 2^-10 descale (half a mantissa step in
    the normal range, half the subnormal step 2^-9 in code units, and the fp32
    roundings of r, descale and x * r). Zeros stay zero, no code is NaN and
    every descale is a positive normal fp32 number."""
    x = _block_of(amax)[None, None]
    codes, ds = quantize(x)
    tab = e4m3_decode_table()
    assert not np.isnan(tab[codes]).any()
    d = float(ds[0, 0, 0])
    assert 2.0 ** -126 <= d < math.inf
    deq = dequantize(codes, ds)
    xf = x.double().numpy()
    assert np.all(deq[xf == 0] == 0)
    bound = (2.0 ** -4 + 2.0 ** -21) * np.abs(xf) + 2.0 ** -10 * d
    assert np.all(np.abs(deq - xf) <= bound)


def test_quantize_tiny_block_rule():
    """0 < amax < 448 * 2^-126: descale 2^-126 and r = 2^126 exactly, so the
    codes are those of x * 2^126 (exact in fp32) and nothing saturates."""
    for amax in (1e-37, 3e-36, 2.0 ** -130):
        x = _block_of(amax, seed=1)[None, None]
        codes, ds = quantize(x)
        assert ds[0, 0, 0] == np.float32(2.0 ** -126)
        y = (x.double() * 2.0 ** 126).float().numpy()
        assert np.array_equal(codes, torch_codes(y))
        assert np.abs(e4m3_decode_table()[codes]).max() < 448.0
    # at amax = 448 * 2^-126 exactly, the ordinary rule gives the same numbers
    x = _block_of(7 * 2.0 ** -120, seed=2)[None, None]
    codes, ds = quantize(x)
    assert ds[0, 0, 0] == np.float32(2.0 ** -126)
    assert np.array_equal(codes, torch_codes((x.double() * 2.0 ** 126).float().numpy()))
    # per tensor: a tiny global amax takes the same rule in every slot
    x = torch.cat([_block_of(1e-37, seed=3), _block_of(2e-38, seed=4)])[None, None]
    _, ds = quantize(x, per_tensor=True)
    assert np.all(ds == np.float32(2.0 ** -126))
