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
"""

import numpy as np


def decode_bf16(bits):
    """bf16 codes (uint16 array) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):    # NaN codes stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_e4m3fn(codes):
    """OCP E4M3FN codes (uint8 array) -> float64, exact; 0x7F and 0xFF give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(e > 0, normal, subnormal)
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)
