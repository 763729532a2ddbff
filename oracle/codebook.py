"""Per-output-channel codebook quantization (LowRA-style).

LowRA page:
  * section 3 (workflow): an output-channel quantization kernel takes custom
    thresholds and a given precision per channel; a per-output-channel
    dequantization kernel recovers the base weight for fine-tuning;
  * section 4.1: each output channel gets its own precision, its own mapping
    (the representative value of each code) and thresholds (the bin edges,
    figure 3); inside a channel, groups of 64 elements are scaled by their
    absmax, following QLoRA.

Readings where the pages are silent:
  * code = number of the row's thresholds strictly below x = w / c (a value on
    a threshold goes to the lower bin), x computed as in NF4;
  * packing: each 64-block of a row with b bits is stored as b bit-planes of
    64 bits; plane p is a little-endian uint64 whose bit e is bit p of the
    code of element e of the block; a block takes 8*b bytes; row i starts at
    byte offset sum over earlier rows of K*b/8;
  * dequant: w' = bfloat16(float32(L_i[code] * c'_j)).
"""
from __future__ import annotations

import numpy as np

from .bf16 import round_bf16, f32_to_bf16_bits
from .nf4 import block_absmax, normalise

BLOCK = 64


def row_offsets(row_bits: np.ndarray, K: int) -> np.ndarray:
    b = np.asarray(row_bits, dtype=np.int64)
    off = np.zeros(b.size + 1, dtype=np.int64)
    off[1:] = np.cumsum(K * b // 8)
    return off


def codes_of_row(x_row: np.ndarray, t_row: np.ndarray, nbits: int) -> np.ndarray:
    code = np.zeros(x_row.shape, dtype=np.uint8)
    for k in range((1 << nbits) - 1):
        code += (x_row > np.float32(t_row[k])).astype(np.uint8)
    return code


def pack_planes(codes_row: np.ndarray, nbits: int, block: int = BLOCK) -> np.ndarray:
    """Bit-plane packing of one row's codes (see module docstring): for each
    block, plane p = the 64 bits (bit p of code e) for e = 0..63, eight bytes,
    least significant bit first."""
    c = np.asarray(codes_row, dtype=np.uint8).reshape(-1, block)
    planes = np.zeros((c.shape[0], nbits, block // 8), dtype=np.uint8)
    for p in range(nbits):
        bitp = (c >> p) & 1
        planes[:, p, :] = np.packbits(bitp, axis=1, bitorder="little")
    return planes.reshape(-1)


def unpack_planes(row_bytes: np.ndarray, nbits: int, K: int, block: int = BLOCK) -> np.ndarray:
    planes = np.asarray(row_bytes, dtype=np.uint8).reshape(K // block, nbits, block // 8)
    codes = np.zeros((K // block, block), dtype=np.uint8)
    for p in range(nbits):
        bits = np.unpackbits(planes[:, p, :], axis=1, bitorder="little")
        codes |= (bits << p).astype(np.uint8)
    return codes.reshape(-1)


def quantize(W: np.ndarray, row_bits: np.ndarray, T: np.ndarray, block: int = BLOCK):
    """W [N, K] float32, row_bits [N] in {1..4}, T [N, 15] float32 (first
    2^b - 1 used, strictly increasing). Returns (packed bytes, absmax [N*K/64],
    codes uint8 [N, K])."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    c = block_absmax(W, block)
    x = normalise(W, c, block).reshape(N, K)
    off = row_offsets(row_bits, K)
    packed = np.zeros(int(off[-1]), dtype=np.uint8)
    codes = np.zeros((N, K), dtype=np.uint8)
    row_bits = np.asarray(row_bits)
    T = np.asarray(T, dtype=np.float32)
    for b in np.unique(row_bits):
        rows = np.nonzero(row_bits == b)[0]
        cb = np.zeros((rows.size, K), dtype=np.uint8)
        for k in range((1 << int(b)) - 1):
            cb += (x[rows] > T[rows, k][:, None]).astype(np.uint8)
        codes[rows] = cb
    for i in range(N):
        packed[off[i]:off[i + 1]] = pack_planes(codes[i], int(row_bits[i]), block)
    return packed, c, codes


def dequant(packed: np.ndarray, row_bits: np.ndarray, L: np.ndarray, cprime: np.ndarray,
            N: int, K: int, block: int = BLOCK, as_bits: bool = False):
    off = row_offsets(row_bits, K)
    cp = np.asarray(cprime, dtype=np.float32).reshape(N, K // block)
    out = np.empty((N, K), dtype=np.float32)
    for i in range(N):
        b = int(row_bits[i])
        codes = unpack_planes(packed[off[i]:off[i + 1]], b, K, block).reshape(-1, block)
        Li = np.asarray(L[i], dtype=np.float32)
        out[i] = (Li[codes] * cp[i][:, None]).reshape(-1)      # float32 multiply
    return f32_to_bf16_bits(out) if as_bits else round_bf16(out)
