"""The 8-bit float used for the second-level constants.

The QLoRA page (section "贡献二：Double Quantization") says the block constants
are quantized again with an 8-bit float, but does not say which one. Reading
taken: OCP 8-bit floating point "E4M3" -- sign, 4 exponent bits (bias 7),
3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448,
subnormals m * 2^-9. Encoding rounds to nearest with ties to the even code,
after the caller has clamped to [-448, 448]; -0 encodes as 0x80.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """Value of each E4M3 code (float32; NaN for 0x7F/0xFF)."""
    code = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(np.float32)


def e4m3_encode(v) -> np.ndarray:
    """E4M3 code of each float32 in [-448, 448], round to nearest even.

    |v| < 2^-6 lies in the subnormal range, where the step is 2^-9, so the
    mantissa is |v| / 2^-9 rounded to the nearest integer (ties to even);
    the result 8 is the smallest normal, whose code is also 8.
    Otherwise |v| = 2^e * (1 + f) with f in [0, 1); the 3-bit mantissa is
    f * 8 rounded to nearest even, carrying into the exponent at 8.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode: input outside [-448, 448]")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    sub = a < 2.0 ** -6
    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range (scaling by a power of two is exact)
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    # normal range
    mant, ex = np.frexp(np.where(sub, 1.0, a))   # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                   # a = 2^e * (2 * mant)
    f = 2.0 * mant - 1.0                         # exact
    m = np.rint(f * 8.0).astype(np.int64)        # exact scaling, rint = ties-to-even
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    normal_code = ((e + 7) << 3) | m
    code = np.where(sub, code, normal_code)
    return (code | sign).astype(np.uint8)
