"""Storage of a quantized weight and its bits per parameter.

QLoRA page, section "贡献二：Double Quantization": one FP32 constant per 64
weights costs 32/64 = 0.5 bit per parameter; after double quantization the
cost is 8/64 + 32/(64*256) ~= 0.127 bit per parameter, 0.373 less, which for
a 30B model saves about 30e9 * 0.373 / 8 ~= 1.40 GB.
"""
from __future__ import annotations

from fractions import Fraction


def storage(N: int, K: int, bits_per_weight=4, block: int = 64, dq_block: int = 256,
            double_quant: bool = True, row_bits=None) -> dict:
    """Byte counts of the quantized representation of an [N, K] weight.

    bits_per_weight: 4 for NF4; for per-channel codebooks pass row_bits.
    The mean of the double quantization is one float32 per tensor.
    """
    n = N * K
    n_b = n // block
    n_d = -(-n_b // dq_block)
    if row_bits is None:
        code_bytes = n * bits_per_weight // 8
    else:
        code_bytes = sum(K * int(b) // 8 for b in row_bits)
    if double_quant:
        const_bytes = n_b + 4 * n_d + 4
    else:
        const_bytes = 4 * n_b
    return {"n": n, "n_blocks": n_b, "n_dq_blocks": n_d,
            "code_bytes": code_bytes, "const_bytes": const_bytes}


def constant_bits_per_param(block: int = 64, dq_block: int = 256, double_quant: bool = True) -> Fraction:
    """Asymptotic constant overhead in bits per parameter (per-tensor terms
    such as the mean vanish)."""
    if not double_quant:
        return Fraction(32, block)
    return Fraction(8, block) + Fraction(32, block * dq_block)


def saving_bytes(n_params: float, block: int = 64, dq_block: int = 256) -> float:
    saved = constant_bits_per_param(block, dq_block, False) - constant_bits_per_param(block, dq_block, True)
    return n_params * float(saved) / 8.0
