"""Stored-format rules for the hot path's caches, written from their definitions.

TEST INFRASTRUCTURE. This module is part of the CPU oracle: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline may import it.  It shares no
code with the HIP path.

Which formats exist comes from the pages only loosely: the b-lab.team summary of
DeepSeek-V4 ("Core Methodological Innovations", item 4, Quantization-Aware
Training bullet) says the indexer query-key path is quantised to FP4.  The exact
encodings below are readings of that statement:

* bf16: round-to-nearest-even from fp32 to an 8-bit significand.
* fp8 e4m3 (OCP "fn" variant, max 448, no infinities): one fp32 scale per row,
  s = amax / 448 computed in fp32 (s = 1 when amax = 0), code = RNE(x / s) with
  the quotient computed in fp32, saturated to +-448.  The division is done in
  fp32 on purpose: a GPU kernel takes the same decision in fp32, and where
  floating point decides an integer code both sides must use one precision.
* MXFP4 (OCP microscaling, v1.0 layout): blocks of 32 consecutive elements share
  an e8m0 scale 2**e with e = floor(log2(amax)) - 2, clamped to [-127, 127]
  (code e + 127; amax = 0 gives code 0 and all-zero elements).  Each element is
  RNE(x / 2**e) on the e2m1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
  code, saturated to +-6; the sign bit is the sign bit of x.  Element 2i is the
  low nibble of byte i.

Every rounding below is done in exact fp64 arithmetic on values that fp64 holds
exactly (fp32 inputs, powers of two), so the decisions are exact.
"""
from __future__ import annotations


import numpy as np

# ----------------------------------------------------------------------------
# generic helper: round a non-negative exact value to a multiple of `quantum`,
# ties to an even multiple.
# ----------------------------------------------------------------------------


def _round_half_even(v: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, ties to even (numpy's rint does exactly this)."""
    return np.rint(v)


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------


def round_bf16(x) -> np.ndarray:
    """fp32 values -> the nearest bf16 value (as fp64), ties to even.

    bf16 keeps fp32's 8 exponent bits and 7 stored significand bits, so in the
    binade [2**e, 2**(e+1)) the spacing is 2**(e-7); below 2**-126 the spacing
    stays 2**-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = np.zeros_like(x)
    a = np.abs(x)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    # log2 may be off by one ulp near powers of two: correct e so 2**e <= a < 2**(e+1)
    e = np.where(np.exp2(e) > a[nz], e - 1, e)
    e = np.where(np.exp2(e + 1) <= a[nz], e + 1, e)
    e = np.maximum(e, -126.0)
    q = np.exp2(e - 7)
    out[nz] = _round_half_even(a[nz] / q) * q
    out = np.where(np.isfinite(x), out, a)
    return np.copysign(out, x)


# ----------------------------------------------------------------------------
# fp8 e4m3 (fn): 1 sign, 4 exponent (bias 7), 3 mantissa; 0x7F/0xFF are NaN.
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> fp64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    mt = c & 0x7
    val = np.where(ex == 0, mt * 2.0 ** -9, (8 + mt) * np.exp2(ex - 10.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_round(y) -> np.ndarray:
    """Exact values -> nearest e4m3 value (fp64), ties to even, saturating at 448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    e = np.where(np.exp2(e) > a[nz], e - 1, e)
    e = np.where(np.exp2(e + 1) <= a[nz], e + 1, e)
    e = np.maximum(e, -6.0)  # below 2**-6 the spacing is the subnormal 2**-9
    q = np.exp2(e - 3)
    out[nz] = _round_half_even(a[nz] / q) * q
    return np.copysign(out, y)


def e4m3_encode_value(v) -> np.ndarray:
    """Values already on the e4m3 grid -> uint8 codes (sign bit from the sign of v)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = (a > 0) & (a < 2.0 ** -6)
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = a >= 2.0 ** -6
    e = np.floor(np.log2(a[nrm]))
    e = np.where(np.exp2(e) > a[nrm], e - 1, e)
    e = np.where(np.exp2(e + 1) <= a[nrm], e + 1, e)
    mant = np.rint(a[nrm] / np.exp2(e - 3)).astype(np.int64) - 8
    code[nrm] = ((e.astype(np.int64) + 7) << 3) | mant
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def quantize_fp8_rows(x):
    """[rows, cols] fp32 -> (codes uint8 [rows, cols], scale float32 [rows]).

    s = fp32(amax / 448) (1 when the row is all zero); code = e4m3(RNE(fp32(x / s))).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / s[..., None]).astype(np.float32)  # fp32 quotient, correctly rounded
    codes = e4m3_encode_value(e4m3_round(y.astype(np.float64)))
    return codes, s


def dequantize_fp8_rows(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# ----------------------------------------------------------------------------
# MXFP4: e2m1 elements with an e8m0 scale per 32 elements
# ----------------------------------------------------------------------------

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def e2m1_decode(nibbles) -> np.ndarray:
    n = np.asarray(nibbles, dtype=np.int64) & 0xF
    mag = E2M1_GRID[n & 0x7]
    return np.where(n & 0x8, -mag, mag)


def e2m1_round_code(v) -> np.ndarray:
    """|v| (exact) -> e2m1 magnitude code 0..7: nearest grid point, ties to the even code,
    saturating at 6."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    # distance to every grid point, pick the nearest; on an exact tie prefer the even code
    d = np.abs(a[..., None] - E2M1_GRID)
    best = np.min(d, axis=-1, keepdims=True)
    cand = d == best
    codes = np.arange(8)
    # among the (one or two) nearest codes choose the even one
    even_pick = np.where(cand & (codes % 2 == 0), codes, 99).min(axis=-1)
    any_pick = np.where(cand, codes, 99).min(axis=-1)
    return np.where(even_pick < 99, even_pick, any_pick)


def mx_scale_exponent(amax) -> np.ndarray:
    """e = floor(log2(amax)) - 2 taken exactly from frexp, clamped to [-127, 127];
    amax = 0 gives -127 (scale code 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)  # amax = f * 2**ex with f in [0.5, 1)  =>  floor(log2) = ex - 1
    e = ex.astype(np.int64) - 1 - 2
    e = np.clip(e, -127, 127)
    return np.where(amax > 0, e, -127)


def quantize_mxfp4(x):
    """[..., n] fp32 with n % 32 == 0 -> (packed codes uint8 [..., n/2], e8m0 scales uint8 [..., n/32])."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = x.shape[-1]
    assert n % MX_BLOCK == 0, "MXFP4 rows must be a multiple of 32 elements"
    blk = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    e = mx_scale_exponent(amax)
    scaled = blk / np.exp2(e.astype(np.float64))[..., None]
    mag = e2m1_round_code(scaled)
    nib = (mag | np.where(np.signbit(blk), 8, 0)).astype(np.uint8)
    nib = np.where((amax > 0)[..., None], nib, 0).astype(np.uint8)
    nib = nib.reshape(x.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


def dequantize_mxfp4(packed, scales) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0xF
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    vals = e2m1_decode(nib)
    e = np.asarray(scales, dtype=np.int64) - 127
    blk = vals.reshape(vals.shape[:-1] + (vals.shape[-1] // MX_BLOCK, MX_BLOCK))
    return (blk * np.exp2(e.astype(np.float64))[..., None]).reshape(vals.shape)

