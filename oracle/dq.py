"""Double quantization of the float32 block constants.

QLoRA page, section "贡献二：Double Quantization":
  * the first-level constants (one FP32 per 64 weights) are treated as a
    second data set and quantized with an 8-bit float at block size 256;
  * the constants are all positive, so their mean is subtracted first (the
    values then straddle zero and use both signs of the symmetric code) and
    added back at dequantization;
  * constant overhead: 8/64 + 32/(64*256) = 0.127 bit per parameter.

Readings where the pages are silent:
  * one mean per tensor -- the 0.127 closed form has exactly one 32-bit term
    per 256 constants, so there is no per-block mean;
  * the mean is the float64 sum of the constants taken as a fixed binary
    tree (pairwise inside each 256-block, then pairwise over the block sums
    padded with zeros to a power of two), divided by their count, rounded
    to float32;
  * the 8-bit float is OCP E4M3, each 256-block scaled so that its largest
    |c - mean| maps to 448; s2 = a2 / 448 in float32; a block with a2 = 0
    stores code 0 and decodes to the mean;
  * decode is one fused multiply-add: c' = fma(E4M3(code), s2, mean).
"""
from __future__ import annotations

import math

import numpy as np

from .bf16 import fma_f32
from .fp8 import e4m3_decode, e4m3_encode, E4M3_MAX

DQ_BLOCK = 256


def pairwise_sum_f64(v: np.ndarray) -> float:
    """Sum of a power-of-two-length float64 vector as a balanced binary tree:
    neighbours are added level by level."""
    v = np.asarray(v, dtype=np.float64)
    assert v.size & (v.size - 1) == 0
    while v.size > 1:
        v = v[0::2] + v[1::2]
    return float(v[0])


def tree_mean(c: np.ndarray, dq_block: int = DQ_BLOCK) -> np.float32:
    c = np.asarray(c, dtype=np.float32)
    n_b = c.size
    n_d = -(-n_b // dq_block)
    padded = np.zeros(n_d * dq_block, dtype=np.float64)
    padded[:n_b] = c
    block_sums = [pairwise_sum_f64(padded[J * dq_block:(J + 1) * dq_block]) for J in range(n_d)]
    width = 1
    while width < n_d:
        width *= 2
    top = np.zeros(width, dtype=np.float64)
    top[:n_d] = block_sums
    S = pairwise_sum_f64(top)
    return np.float32(S / n_b)


def double_quant(absmax: np.ndarray, dq_block: int = DQ_BLOCK):
    """Returns (code8 uint8 [n_b], s2 float32 [n_d], mean float32)."""
    c = np.asarray(absmax, dtype=np.float32)
    n_b = c.size
    n_d = -(-n_b // dq_block)
    mu = tree_mean(c, dq_block)
    d = (c - mu).astype(np.float32)                       # float32 subtraction
    code8 = np.zeros(n_b, dtype=np.uint8)
    s2 = np.zeros(n_d, dtype=np.float32)
    for J in range(n_d):
        dJ = d[J * dq_block:(J + 1) * dq_block]
        a2 = np.float32(np.max(np.abs(dJ)))
        s2[J] = np.float32(a2 / np.float32(E4M3_MAX))
        if s2[J] > 0:
            v = (dJ / s2[J]).astype(np.float32)           # float32 division
            v = np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32)
            code8[J * dq_block:(J + 1) * dq_block] = e4m3_encode(v)
        # else: codes stay 0 (decode to the mean)
    return code8, s2, mu


def dq_decode(code8: np.ndarray, s2: np.ndarray, mu, dq_block: int = DQ_BLOCK) -> np.ndarray:
    """c'_j = fma(E4M3^-1(code8_j), s2_J, mean), J = j // 256."""
    code8 = np.asarray(code8, dtype=np.uint8)
    scale = np.repeat(np.asarray(s2, dtype=np.float32), dq_block)[:code8.size]
    return fma_f32(e4m3_decode(code8), scale, np.float32(mu))


def exact_mean_f32(c: np.ndarray) -> float:
    """Correctly rounded mean (math.fsum is exact) -- for the pin only."""
    return math.fsum(float(x) for x in np.asarray(c, dtype=np.float32)) / len(c)
