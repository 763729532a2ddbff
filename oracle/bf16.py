"""bfloat16 rounding and an fp32 fused multiply-add, written out from the
IEEE definitions.

The QLoRA page (introduction) says the 4-bit base weight is dequantized to
BFloat16 at use time, so the dequantized weight is the bfloat16 value nearest
(ties to even) to the float32 product.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return
    the 16-bit patterns. bfloat16 is the upper half of a float32, so rounding
    keeps the top 16 bits and rounds on the 16 dropped ones."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x) -> np.ndarray:
    """float32 -> nearest bfloat16, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def fma_f32(a, b, c) -> np.ndarray:
    """Single-rounding float32 a*b + c.

    a*b of two float32 values is exact in float64 (24 + 24 <= 53 bits). The
    float64 sum s = a*b + c can round; the exact error e of that addition is
    recovered with Knuth's TwoSum. When e != 0, s is nudged one float64 ulp
    toward e if its last bit is even ("round to odd"). A float64 value rounded
    to odd carries 53 >= 24 + 2 bits, so its nearest-even rounding to float32
    equals the correctly rounded float32 of the exact a*b + c.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    shape = np.broadcast(a, b, c).shape
    p = np.broadcast_to(a * b, shape).reshape(-1)
    cc = np.broadcast_to(c, shape).reshape(-1)
    s = p + cc
    bb = s - p
    err = (p - (s - bb)) + (cc - bb)
    even = (s.view(np.uint64) & np.uint64(1)) == 0
    fix = (err != 0) & even
    if np.any(fix):
        s[fix] = np.nextafter(s[fix], np.where(err[fix] > 0, np.inf, -np.inf))
    return s.astype(np.float32).reshape(shape)
