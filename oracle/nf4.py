"""NF4: the 16-level NormalFloat table, blockwise absmax quantization,
nibble packing and dequantization.

QLoRA page, section "贡献一：4-bit NormalFloat（NF4）":
  * the 16 candidate values sit at standard-normal quantiles so that each
    bin holds about the same probability mass, denser near 0;
  * the weights of a block are divided by the block's absolute maximum,
    which scales them into [-1, 1], and each is mapped to the nearest NF4
    value; the 4-bit index and the block constant are stored;
  * exact zero is kept by taking 8 quantiles for the negative half and 9 for
    the positive half and dropping the duplicated 0: 8 + 9 - 1 = 16.
Section "贡献二：Double Quantization": one FP32 constant per 64 weights.

Readings where the page is silent:
  * truncation probability delta = 1 - (1/32 + 1/30)/2 (not on the page);
  * quantiles equally spaced in probability on each half;
  * ties at a midpoint go to the lower index: thresholds are the float32
    midpoints rounded toward -inf, and a code counts thresholds strictly
    below x;
  * normalisation is an IEEE float32 division; an all-zero block gives x = +0;
  * packing: byte e/2 holds element e (even) in bits 7..4, element e+1 in 3..0.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
from scipy.special import ndtri

from .bf16 import round_bf16, f32_to_bf16_bits

BLOCK = 64
DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def quantile_probs(delta: float, n_steps: int) -> np.ndarray:
    """n_steps + 1 probabilities from 1/2 to delta in equal steps."""
    return np.array([0.5 + (delta - 0.5) * (j / n_steps) for j in range(n_steps + 1)])


def levels_f64(delta: float = DELTA, half: int = 8) -> np.ndarray:
    """The 2*half levels in float64, ascending, normalised to [-1, 1].

    Positive half: half + 1 quantiles Phi^-1(p), p from 1/2 to delta, the first
    being 0. Negative half: half quantiles -Phi^-1(p), p from 1/2 to delta,
    the first being 0. Both are divided by Phi^-1(delta), so the extreme
    levels are exactly -1 and +1; the duplicate 0 of the negative half is
    dropped. For half = 8 this is NF4 (8 + 9 - 1 = 16).
    """
    scale = ndtri(delta)
    pos = [ndtri(p) / scale for p in quantile_probs(delta, half)]
    neg = [-ndtri(p) / scale for p in quantile_probs(delta, half - 1)]
    assert pos[0] == 0.0 and neg[0] == 0.0
    vals = [0.0] + pos[1:] + neg[1:]
    vals.sort()
    return np.array(vals, dtype=np.float64)


def levels(delta: float = DELTA) -> np.ndarray:
    """NF4 levels q_0 < ... < q_15 rounded to float32."""
    return levels_f64(delta).astype(np.float32)


def round_down_f32(m: float) -> np.float32:
    """Largest float32 <= m (m a float64)."""
    f = np.float32(m)
    if float(f) > m:
        f = np.nextafter(f, np.float32(-np.inf))
    return np.float32(f)


def midpoint_thresholds(q: np.ndarray) -> np.ndarray:
    """t_i = largest float32 <= (q_i + q_{i+1}) / 2. The sum of two float32
    values and its halving are exact in float64."""
    q = np.asarray(q, dtype=np.float32)
    return np.array([round_down_f32((float(q[i]) + float(q[i + 1])) / 2.0)
                     for i in range(len(q) - 1)], dtype=np.float32)


def thresholds(delta: float = DELTA) -> np.ndarray:
    return midpoint_thresholds(levels(delta))


def block_absmax(W: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """c_j = max |w| over each run of `block` consecutive elements (row-major
    flat order); W's last dimension must be a multiple of `block`."""
    W = np.asarray(W, dtype=np.float32)
    assert W.shape[-1] % block == 0
    return np.abs(W.reshape(-1, block)).max(axis=1)


def normalise(W: np.ndarray, absmax: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """x = w / c_j in float32 (IEEE division); x = +0 where c_j == 0."""
    blocks = np.asarray(W, dtype=np.float32).reshape(-1, block)
    c = np.asarray(absmax, dtype=np.float32)
    x = np.zeros(blocks.shape, dtype=np.float32)
    nz = c > 0
    x[nz] = blocks[nz] / c[nz, None]
    return x.reshape(-1)


def count_above(x: np.ndarray, t: np.ndarray) -> np.ndarray:
    """code = number of thresholds strictly below x."""
    code = np.zeros(x.shape, dtype=np.uint8)
    for ti in np.asarray(t, dtype=np.float32):
        code += (x > ti).astype(np.uint8)
    return code


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    assert c.size % 2 == 0
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(2 * p.size, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0xF
    return out


def quantize(W: np.ndarray, block: int = BLOCK, t: np.ndarray = None):
    """Blockwise NF4 quantization of W [N, K] (float32).

    Returns (packed codes uint8 [N*K/2], absmax float32 [N*K/64]).
    """
    t = thresholds() if t is None else t
    c = block_absmax(W, block)
    x = normalise(W, c, block)
    codes = count_above(x, t)
    return pack_nibbles(codes), c


def dequant(packed: np.ndarray, cprime: np.ndarray, shape, block: int = BLOCK,
            q: np.ndarray = None, as_bits: bool = False):
    """w' = bfloat16(float32(q[code] * c'_j)) with c' the (possibly double
    quantized) block constant. Returns float32 values, or bf16 bits."""
    q = levels() if q is None else np.asarray(q, dtype=np.float32)
    codes = unpack_nibbles(packed).reshape(-1, block)
    prod = q[codes] * np.asarray(cprime, dtype=np.float32)[:, None]   # float32 multiply
    prod = prod.reshape(shape)
    return f32_to_bf16_bits(prod) if as_bits else round_bf16(prod)


def nearest_code_bruteforce(x: np.ndarray, q: np.ndarray = None) -> np.ndarray:
    """argmin_i |x - q_i| in exact rational arithmetic, ties to the lower
    index. Slow; for pins on small inputs."""
    q = levels() if q is None else q
    qf = [Fraction(float(v)) for v in q]
    out = np.empty(len(x), dtype=np.uint8)
    for n, xv in enumerate(np.asarray(x, dtype=np.float32)):
        xf = Fraction(float(xv))
        best, bi = None, 0
        for i, qi in enumerate(qf):
            d = abs(xf - qi)
            if best is None or d < best:
                best, bi = d, i
        out[n] = bi
    return out


def roundtrip_error(W: np.ndarray, block: int = BLOCK) -> float:
    """AQLoRA page, section 3.1: eps = (1/|W|) * sum over blocks of the squared
    L2 distance between a block and its absmax-NF4 round trip. The round
    trip here keeps the float32 constant (no double quantization) and the
    float32 product before bfloat16 rounding, as the section describes the
    quantizer alone."""
    packed, c = quantize(W, block)
    q = levels()
    codes = unpack_nibbles(packed).reshape(-1, block)
    rec = (q[codes] * c[:, None]).astype(np.float64)
    diff = np.asarray(W, dtype=np.float64).reshape(-1, block) - rec
    return float(np.sum(diff * diff) / diff.size)


TAU = 0.01   # AQLoRA page, section 3.1: threshold of the small-weight fraction


def small_fraction(W: np.ndarray, tau: float = TAU) -> float:
    """AQLoRA page, section 3.1: s = Pr[|w| < tau] over the layer's weights.
    The comparison is exact: |w| (a float32 value) against tau in float64."""
    a = np.abs(np.asarray(W, dtype=np.float32).astype(np.float64))
    return float(np.count_nonzero(a < tau)) / a.size


def profile(W: np.ndarray, tau: float = TAU, block: int = BLOCK):
    """The AQLoRA profiling pass of one layer (section 3.1): returns
    (eps, s) = (mean squared NF4 round-trip error, small-weight fraction)."""
    return roundtrip_error(W, block), small_fraction(W, tau)
