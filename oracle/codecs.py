"""Exact decoders for the two storage formats, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the upper 16 bits of an IEEE-754 binary32 word, so a code c decodes
  to the binary32 whose bit pattern is c << 16.
* FP8 E4M3 ("E4M3FN" in the OCP 8-bit floating point specification): 1 sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 holds
  subnormals, (-1)^s * 2^-6 * m/8.  There is no infinity; the two codes with
  all exponent and mantissa bits set (0x7F, 0xFF) are NaN, so the largest
  finite magnitude is 2^8 * 1.75 = 448.  The FP8 KV cache on the
  "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000" page (intro and
  "What the kernels do") stores this format.

encode_e4m3fn is the plain definition of round-to-nearest-even onto the
finite E4M3FN values, after clamping the magnitude to 448.
"""

import numpy as np


def decode_bf16(bits):
    """bf16 codes (uint16 array) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):    # NaN codes stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3fn_value(c):
    """The value of each E4M3FN code in c (int64 array) from the format's fields."""
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(e > 0, normal, subnormal)
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


# All 256 codes' values, evaluated once from the fields above: decoding a
# large cache is then one table lookup per code (same values).
_E4M3_VALUES = _e4m3fn_value(np.arange(256, dtype=np.int64))


def decode_e4m3fn(codes):
    """OCP E4M3FN codes (uint8 array) -> float64, exact; 0x7F and 0xFF give NaN."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


# The 127 non-negative finite E4M3FN values, in code order (ascending).
_E4M3_GRID = None


def encode_e4m3fn(x):
    """float32 array -> OCP E4M3FN codes (uint8): round to nearest even.

    Magnitudes above 448 (infinity included) clamp to 448; NaN maps to the
    NaN code 0x7F with the input's sign bit.  The nearest of the finite
    values is chosen; on a tie the even code wins, which is the even
    mantissa, since consecutive codes are consecutive values and a code's
    last bit is its mantissa's last bit.  The sign bit is copied (so -0.0
    encodes as 0x80).
    """
    global _E4M3_GRID
    if _E4M3_GRID is None:
        _E4M3_GRID = decode_e4m3fn(np.arange(127, dtype=np.uint8))
    grid = _E4M3_GRID
    v = np.asarray(x, dtype=np.float32)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, 448.0))
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)     # first value >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = (d_hi == d_lo) & (hi != lo)
    pick = np.where(tie, np.where(hi % 2 == 0, hi, lo), pick)
    pick = np.where(a == grid[hi], hi, pick)                          # exact values
    codes = pick.astype(np.uint8) | sign
    return np.where(nan, np.uint8(0x7F) | sign, codes).astype(np.uint8)
