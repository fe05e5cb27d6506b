"""Pins of the MXFP8 oracle against what the format itself fixes (OCP Microscaling Formats v1.0,
MXFP8 with E4M3 elements) rather than against the oracle's own formulas."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import mxfp8 as MX


def _e4m3_table() -> np.ndarray:
    """Every finite non-negative E4M3 value, built from the bit fields by hand: subnormals
    m * 2**-9 (m = 1..7) and normals (1 + m/8) * 2**(e-7) for e = 1..15, except the NaN code."""
    vals = [0.0] + [m * 2.0 ** -9 for m in range(1, 8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(sorted(vals))


def _nearest_even_brute(y: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Nearest table value by exhaustive search; exact ties go to the value whose code is even
    (mantissa LSB 0), magnitudes beyond the largest value saturate."""
    out = np.empty_like(y)
    codes = np.arange(len(table))  # table index = code for non-negative values
    for i, v in enumerate(y):
        a = abs(v)
        if a >= table[-1]:
            r = table[-1]
        else:
            d = np.abs(table - a)
            best = np.flatnonzero(d == d.min())
            r = table[best[0]] if len(best) == 1 else table[best[codes[best] % 2 == 0][0]]
        out[i] = np.copysign(r, v)
    return out


def test_table_matches_decode_of_every_code():
    table = _e4m3_table()
    assert len(table) == 127 and table[-1] == 448.0 and table[1] == 2.0 ** -9
    dec = MX.e4m3_decode(np.arange(127, dtype=np.uint8))
    np.testing.assert_array_equal(dec, table)
    assert np.isnan(MX.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    np.testing.assert_array_equal(MX.e4m3_decode(np.arange(128, 255, dtype=np.uint8)), -table)


def test_round_matches_brute_force_nearest_even():
    rng = np.random.default_rng(1)
    table = _e4m3_table()
    mids = (table[1:] + table[:-1]) / 2                     # every exact tie
    y = np.concatenate([rng.uniform(-500, 500, 2000), rng.uniform(-0.05, 0.05, 2000),
                        rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 9, 2000),
                        mids, -mids, table, -table, [0.0, -0.0, 460.0, 464.0, 479.0, 1e6]])
    np.testing.assert_array_equal(MX.e4m3_round(y), _nearest_even_brute(y, table))


def test_fixed_points_of_the_format():
    r = MX.e4m3_round
    assert r(np.array([448.0]))[0] == 448.0
    assert r(np.array([1000.0]))[0] == 448.0                 # saturation
    assert r(np.array([2.0 ** -10]))[0] == 0.0               # tie between 0 and 2**-9 -> 0 (even)
    assert r(np.array([3 * 2.0 ** -10]))[0] == 2 * 2.0 ** -9  # tie between codes 1 and 2 -> 2
    assert r(np.array([1.0 + 1 / 16]))[0] == 1.0               # tie between 1 and 1.125 -> 1
    assert r(np.array([1.0 + 3 / 16]))[0] == 1.25              # tie between 1.125 and 1.25 -> 1.25
    np.testing.assert_array_equal(MX.e4m3_encode(np.array([448.0, 1.0, 2.0 ** -9, 2.0 ** -6, -2.0])),
                                  np.array([0x7E, 0x38, 0x01, 0x08, 0xC0], np.uint8))


def test_scale_is_tight_and_errors_within_the_rounding_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-20, 20, (64, 1))
    x[3, 32:64] = 0.0                                         # one all-zero block
    codes, scales = MX.mx_quantize_rows(x)
    assert codes.shape == (64, 256) and scales.shape == (64, 8)
    deq = MX.mx_dequantize_rows(codes, scales)
    blocks = np.abs(x).reshape(64, 8, 32)
    amax = blocks.max(axis=2)
    e = scales.astype(np.int64) - 127
    nz = amax > 0
    # the block maximum lands in [256, 512) before rounding: the largest code is >= 256
    top = np.abs(MX.e4m3_decode(codes)).reshape(64, 8, 32).max(axis=2)
    assert np.all((amax[nz] / np.exp2(e[nz]) >= 256) & (amax[nz] / np.exp2(e[nz]) < 512))
    assert np.all(top[nz] >= 256)
    assert scales[3, 1] == 0 and np.all(codes[3, 32:64] == 0)
    # per element: half a spacing (|y|/16 for normals, 2**-10 for subnormals) or the saturation
    # step at the top binade (|y|/8), in units of the block scale
    y = np.abs(x).reshape(64, 8, 32) / np.exp2(e)[:, :, None]
    err = np.abs(deq - x).reshape(64, 8, 32) / np.exp2(e)[:, :, None]
    bound = np.maximum(np.where(y >= 448, y / 8, y / 16), 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))


def test_blocks_on_the_grid_round_trip_exactly_and_integer_products_are_exact():
    rng = np.random.default_rng(3)
    # every element a small integer times the block's power of two, block max exactly 256 * 2**s
    s = rng.integers(-30, 30, (16, 4))
    ints = rng.integers(-15, 16, (16, 4, 32)).astype(np.float64)
    ints[:, :, 0] = 256.0
    x = (ints * np.exp2(s)[:, :, None]).reshape(16, 128)
    codes, scales = MX.mx_quantize_rows(x)
    np.testing.assert_array_equal(scales.astype(np.int64) - 127, s)
    np.testing.assert_array_equal(MX.mx_dequantize_rows(codes, scales), x)
    w = rng.integers(-15, 16, (8, 128)).astype(np.float64)
    w[:, ::32] = 256.0
    wc, ws = MX.mx_quantize_rows(w)
    C = MX.mx_grouped_gemm_rows(codes, scales, wc[None], ws[None], np.array([0, 16]))
    np.testing.assert_array_equal(C, x @ w.T)               # every term exact in float64


def test_padding_and_grouped_column_layout():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 40))                        # K = 40 pads to 64
    codes, scales = MX.mx_quantize_rows(x)
    assert codes.shape == (10, 64) and np.all(codes[:, 40:] == 0)
    # grouped along rows with ragged lengths (including an empty group), stored transposed
    y = rng.standard_normal((70, 6))
    offs = np.array([0, 33, 33, 70])
    c, s, kbase = MX.mx_quantize_grouped_cols(y, offs, 64)
    np.testing.assert_array_equal(kbase, [0, 64, 64, 128])
    c0, s0 = MX.mx_quantize_rows(y[0:33].T)
    np.testing.assert_array_equal(c[:, 0:33], c0[:, 0:33])
    assert np.all(c[:, 33:64] == 0)
    np.testing.assert_array_equal(s[:, 0:1], s0[:, 0:1])
    # the grouped K product equals per-group products of the dequantized segments
    Cg = MX.mx_grouped_gemm_k(c, s, c, s, kbase)
    d = MX.mx_dequantize_rows(c, s)
    np.testing.assert_allclose(Cg[2], d[:, 64:128] @ d[:, 64:128].T, rtol=0, atol=0)
    assert np.all(Cg[1] == 0)


def test_a_planted_exponent_mistake_is_caught(monkeypatch):
    """An off-by-one in the shared exponent (emax 7 instead of 8) must fail the tightness pin."""
    monkeypatch.setattr(MX, "E4M3_EMAX", 7)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 64))
    codes, scales = MX.mx_quantize_rows(x)
    amax = np.abs(x).reshape(8, 2, 32).max(axis=2)
    ratio = amax / np.exp2(scales.astype(np.int64) - 127)
    with pytest.raises(AssertionError):
        assert np.all((ratio >= 256) & (ratio < 512))
