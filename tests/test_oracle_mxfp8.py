"""Pins of the MX-FP8 quantiser oracle (oracle/mxfp8.py) against what the e4m3
and MX definitions fix: every code decodes to its defining value, the encoder
is the nearest-value (ties-to-even) rounding found by brute force over all
codes, scales are powers of two that put the block maximum in [256, 512),
and the round trip stays within half a grid step."""
import numpy as np
import pytest

from oracle import mxfp8 as Q


def all_finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_decode_matches_the_format_definition():
    v = Q.e4m3_decode(all_finite_codes())
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert Q.e4m3_decode([0x38])[0] == 1.0 and Q.e4m3_decode([0x01])[0] == 2.0 ** -9  # 1.0, min subnormal
    assert Q.e4m3_decode([0x08])[0] == 2.0 ** -6 and Q.e4m3_decode([0x7E])[0] == 448.0
    assert np.isnan(Q.e4m3_decode([0x7F, 0xFF])).all()
    pos = np.sort(Q.e4m3_decode(np.arange(0, 0x7F)))
    assert np.all(np.diff(pos) > 0)                       # 127 distinct non-negative values
    assert len(np.unique(v)) == 253                       # +-0 collapse: 254 codes -> 253 values


def test_encoder_is_nearest_even_by_brute_force():
    grid = Q.e4m3_decode(np.arange(0, 0x7F))           # 0 .. 448, ascending
    codes = np.arange(0, 0x7F)
    rng = np.random.default_rng(0)
    q = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 2.0 ** -5, 5000),
                        (grid[1:] + grid[:-1]) / 2])       # include every midpoint (ties)
    got = Q.e4m3_encode(q)
    d = np.abs(q[:, None] - grid[None, :])
    best = d.min(1, keepdims=True)
    cand = np.where(d == best, codes[None, :], 999)
    # ties go to the even mantissa (code's lowest bit 0)
    tie = (d == best).sum(1) > 1
    ref = np.where(tie, np.where(cand % 2 == 0, cand, 999).min(1), cand.min(1))
    np.testing.assert_array_equal(got, ref.astype(np.uint8))
    np.testing.assert_array_equal(Q.e4m3_encode(-q), ref.astype(np.uint8) | 0x80)  # sign bit only


def test_scales_put_block_max_in_range_and_round_trip_is_half_a_step():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :32] = 0.0                                         # an all-zero block
    codes, scales = Q.mx_quantize(x)
    assert codes.shape == x.shape and scales.shape == (64, 8)
    amax = np.abs(x.reshape(64, 8, 32)).max(-1)
    X = 2.0 ** (scales.astype(np.float64) - 127)
    nz = amax > 0
    assert np.all((amax[nz] / X[nz] >= 256) & (amax[nz] / X[nz] < 512))
    assert scales[3, 0] == 127 and np.all(codes[3, :32] == 0)
    y = Q.mx_dequantize(codes, scales)
    xb, yb = x.reshape(64, 8, 32).astype(np.float64), y.reshape(64, 8, 32)
    # error <= half a step of the element's own binade (2^-4 relative) or of the subnormal grid,
    # except saturated elements (clamped to 448 X)
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(xb) / X[..., None], 1e-300))) - 3), 2.0 ** -9)
    sat = np.abs(xb) / X[..., None] > 448
    err = np.abs(xb - yb) / X[..., None]
    assert np.all(err[~sat] <= step[~sat] / 2 * (1 + 1e-12))
    assert np.all(np.abs(yb[sat]) == 448 * np.broadcast_to(X[..., None], xb.shape)[sat])


def test_scaled_dot_products_track_exact_ones():
    """A product of MX-quantised operands (the FP8 GEMM's arithmetic) is within a few
    percent of the exact product for random data: the bound the slices are held to."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((64, 1536)).astype(np.float32)
    w = (rng.standard_normal((96, 1536)) * 0.02).astype(np.float32)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    got = Q.mx_dequantize(*Q.mx_quantize(a)) @ Q.mx_dequantize(*Q.mx_quantize(w)).T
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel < 0.05
