"""Pins for the oracle's stored-format rules (bf16, fp8 e4m3 + row scale, MXFP4).

Each check ties the oracle to something other than itself: torch's casts (a
library routine), exhaustive code grids, exact midpoints, and frexp.
"""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F


def _interesting_f32(n=20000, seed=7):
    r = np.random.default_rng(seed)
    x = r.standard_normal(n).astype(np.float32) * np.exp2(r.integers(-30, 30, n)).astype(np.float32)
    extra = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 2.0 ** -130, 3.0e38, -3.0e38,
                      1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7], dtype=np.float32)
    return np.concatenate([x, extra])


def test_bf16_matches_torch_cast():
    x = _interesting_f32()
    ours = F.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)


def test_bf16_ties_to_even():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7: even significand wins (1.0)
    assert F.round_bf16(np.float32(1 + 2 ** -8)) == 1.0
    # 1 + 3*2^-8 is the midpoint between 1+2^-7 (odd) and 1+2^-6 (even)
    assert F.round_bf16(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2  # 0x7F and 0xFF


def test_e4m3_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    assert np.array_equal(F.e4m3_round(vals), vals)
    back = F.e4m3_encode_value(vals)
    # +0 and -0 keep their sign bit
    assert np.array_equal(back, codes)


def test_e4m3_round_matches_torch_after_clamp():
    r = np.random.default_rng(3)
    y = (r.standard_normal(50000) * np.exp2(r.integers(-12, 9, 50000))).astype(np.float32)
    y = np.clip(y, -448, 448)
    ours = F.e4m3_round(y.astype(np.float64))
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_midpoints_and_saturation():
    assert F.e4m3_round(1 + 1 / 16) == 1.0      # midpoint 1 | 1.125 -> even (1.0)
    assert F.e4m3_round(1 + 3 / 16) == 1.25     # midpoint 1.125 | 1.25 -> even (1.25)
    assert F.e4m3_round(2.0 ** -10) == 0.0      # half the smallest subnormal -> 0
    assert F.e4m3_round(3 * 2.0 ** -10) == 2 * 2.0 ** -9
    assert F.e4m3_round(500.0) == 448.0
    assert F.e4m3_round(-1e30) == -448.0


def test_fp8_rows_scale_and_bound():
    r = np.random.default_rng(11)
    x = r.standard_normal((64, 512)).astype(np.float32) * 3
    x[5] = 0.0
    codes, s = F.quantize_fp8_rows(x)
    assert s.dtype == np.float32
    assert s[5] == 1.0 and np.all(codes[5] == 0)
    amax = np.abs(x).max(axis=1)
    np.testing.assert_array_equal(s[np.arange(64) != 5], (amax / np.float32(448))[np.arange(64) != 5])
    deq = F.dequantize_fp8_rows(codes, s)
    # RNE error is at most half a grid step: 2^-4 relative in the normal range,
    # 2^-10 * s absolute in the subnormal range
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-12)
    assert np.all(err <= bound)
    # the row maximum lands on +-448
    i = np.argmax(np.abs(x[0]))
    assert abs(F.e4m3_decode(codes[0, i])) == 448.0


def test_e2m1_grid_and_ties():
    n = np.arange(16)
    vals = F.e2m1_decode(n)
    assert list(vals[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    mids = {0.25: 0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0, 7.0: 6.0, 100.0: 6.0}
    for v, want in mids.items():
        assert F.E2M1_GRID[F.e2m1_round_code(v)] == want, v
    # exact grid values map to themselves
    for c, v in enumerate(F.E2M1_GRID):
        assert F.e2m1_round_code(v) == c


def test_mx_scale_exponent_vs_frexp_and_brute_force():
    r = np.random.default_rng(5)
    amax = np.abs(r.standard_normal(5000) * np.exp2(r.integers(-40, 40, 5000)))
    amax = amax.astype(np.float32).astype(np.float64)
    e = F.mx_scale_exponent(amax)
    for a, ee in zip(amax[:500], e[:500]):
        # brute force: the largest integer f with 2**f <= a, minus 2
        f = 0
        while 2.0 ** f > a:
            f -= 1
        while 2.0 ** (f + 1) <= a:
            f += 1
        assert ee == f - 2
        assert ee == math.frexp(a)[1] - 3
    assert F.mx_scale_exponent(0.0) == -127


def test_mxfp4_packing_order_and_zero_block():
    x = np.zeros(64, dtype=np.float32)
    x[0] = 1.0   # element 0 -> low nibble of byte 0
    x[1] = -6.0  # element 1 -> high nibble of byte 0
    x[3] = 0.5
    packed, scales = F.quantize_mxfp4(x)
    # block 0: amax = 6 -> e = floor(log2 6) - 2 = 0 -> scale code 127
    assert scales[0] == 127
    assert packed[0] == (0x2 | (0xF << 4))  # 1.0 is code 2; -6 is 8|7
    assert packed[1] == (0x1 << 4)          # element 3 = 0.5 -> code 1, high nibble
    # block 1 all zero
    assert scales[1] == 0 and np.all(packed[16:] == 0)


def test_mxfp4_round_trip_error_bound():
    r = np.random.default_rng(9)
    x = r.standard_normal((100, 64)).astype(np.float32)
    packed, scales = F.quantize_mxfp4(x)
    deq = F.dequantize_mxfp4(packed, scales)
    e = scales.astype(np.int64) - 127
    step = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)
    # within the block's range the grid spacing is at most 2 * 2^e, so the error is
    # at most one grid unit (2^e); values above 6 * 2^e saturate (at most 2 * 2^e off)
    assert np.all(np.abs(deq - x) <= 2 * step)
    # every dequantised value lies on the scaled grid
    g = np.abs(deq) / step
    assert np.all(np.isin(g, F.E2M1_GRID))


def test_mxfp4_exact_values_survive():
    # values that are exactly grid points times a common power of two survive exactly
    grid = np.array([0.5, 1, 1.5, 2, 3, 4, 6, -6] * 4, dtype=np.float32) * np.float32(2.0 ** -5)
    packed, scales = F.quantize_mxfp4(grid)
    assert np.array_equal(F.dequantize_mxfp4(packed, scales), grid.astype(np.float64))
