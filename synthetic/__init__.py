"""Seeded synthetic inputs for the quantized-LoRA layer workloads.

This module only draws random numbers and lays them out in the shapes of the
workloads. It holds none of the method's arithmetic (no quantization, no
codebook learning, no GEMM), so both the CPU oracle and the HIP library can be
fed from it.

Recipe (every tensor):
  * generator: NumPy ``default_rng(seed)`` (PCG64), ``standard_normal`` in
    float64, scaled by the stated standard deviation, then cast;
  * seed = 1000 * workload_id + tensor_id with tensor ids
    W = 0, X = 1, A = 2, B = 3, G = 4, per-row sigma = 5;
  * W is float32; X, A, B, G are rounded to bfloat16 (round to nearest even)
    and handed out both as raw uint16 bits and as the exactly equal float32.

The shapes stand in for Llama-family linear layers (widths 4096 / 11008 /
28672 x 8192); real checkpoints and datasets are not needed because the
quantizer is data-free.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

TENSOR_ID = {"W": 0, "X": 1, "A": 2, "B": 3, "G": 4, "sigma": 5}


def seed_of(workload_id: int, tensor: str) -> int:
    return 1000 * int(workload_id) + TENSOR_ID[tensor]


def normal(shape, std: float, seed: int) -> np.ndarray:
    """float64 N(0, std^2) draws from PCG64 seeded with ``seed``."""
    rng = np.random.default_rng(seed)
    out = rng.standard_normal(size=shape, dtype=np.float64)
    out *= std
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Input preparation: float -> bfloat16 bit pattern, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Bf16Tensor:
    bits: np.ndarray  # uint16
    f32: np.ndarray   # float32, exactly the bf16 values

    @property
    def shape(self):
        return self.bits.shape


def bf16_normal(shape, std: float, seed: int) -> Bf16Tensor:
    bits = to_bf16_bits(normal(shape, std, seed).astype(np.float32))
    return Bf16Tensor(bits, bf16_bits_to_f32(bits))


@dataclasses.dataclass(frozen=True)
class Layer:
    """One quantized linear layer with a LoRA adapter."""
    name: str
    workload_id: int
    N: int              # output features (rows of W)
    K: int              # input features
    M: int              # tokens
    r: int
    alpha: float
    w_std: float = 0.02
    blocksize: int = 64
    dq_blocksize: int = 256

    @property
    def scale(self) -> float:
        return self.alpha / self.r


# The five workloads (M for the decode GEMV is the largest token count; the
# smaller ones take the first rows of the same X).
LAYERS: Dict[str, Layer] = {
    "linear1k": Layer("linear1k", 1, 1024, 1024, 16, 16, 32.0),
    "q_proj": Layer("q_proj", 2, 4096, 4096, 2048, 16, 32.0),
    "mlp_up": Layer("mlp_up", 3, 11008, 4096, 4096, 64, 16.0),
    "mlp_down": Layer("mlp_down", 30, 4096, 11008, 4096, 64, 16.0),
    "decode": Layer("decode", 4, 28672, 8192, 16, 16, 32.0),
    "lowra": Layer("lowra", 5, 4096, 4096, 2048, 16, 32.0),
}
DECODE_TOKENS = (1, 4, 16)

# Bit mix of the per-output-channel workload, by descending channel sigma:
# 256 rows x 4 bits, 512 x 3, 1280 x 2, 2048 x 1 (average exactly 1.75).
LOWRA_BIT_MIX: List[Tuple[int, int]] = [(256, 4), (512, 3), (1280, 2), (2048, 1)]


def weight(layer: Layer, rows: Optional[slice] = None) -> np.ndarray:
    """W [N, K] float32 ~ N(0, 0.02^2); the per-channel workload scales row i
    by sigma_i / 0.02 with sigma_i = 0.02 * exp(0.3 * z_i)."""
    w = normal((layer.N, layer.K), layer.w_std, seed_of(layer.workload_id, "W"))
    if layer.name == "lowra":
        w *= row_sigma(layer)[:, None] / layer.w_std
    w = w.astype(np.float32)
    return w if rows is None else np.ascontiguousarray(w[rows])


def row_sigma(layer: Layer) -> np.ndarray:
    z = normal((layer.N,), 1.0, seed_of(layer.workload_id, "sigma"))
    return layer.w_std * np.exp(0.3 * z)


def lowra_row_bits(layer: Layer) -> np.ndarray:
    """Per-row bit widths: more bits for the rows with the largest sigma (the
    squared error of a row grows with sigma^2). Stands in for an allocator."""
    sig = row_sigma(layer)
    order = np.argsort(-sig, kind="stable")
    bits = np.empty(layer.N, dtype=np.uint8)
    pos = 0
    for count, b in LOWRA_BIT_MIX:
        bits[order[pos:pos + count]] = b
        pos += count
    assert pos == layer.N
    return bits


def activations(layer: Layer, M: Optional[int] = None) -> Bf16Tensor:
    M = layer.M if M is None else M
    full = bf16_normal((layer.M, layer.K), 1.0, seed_of(layer.workload_id, "X"))
    if M == layer.M:
        return full
    return Bf16Tensor(np.ascontiguousarray(full.bits[:M]), np.ascontiguousarray(full.f32[:M]))


def lora_a(layer: Layer) -> Bf16Tensor:
    return bf16_normal((layer.r, layer.K), 0.02, seed_of(layer.workload_id, "A"))


def lora_b(layer: Layer) -> Bf16Tensor:
    return bf16_normal((layer.N, layer.r), 0.02, seed_of(layer.workload_id, "B"))


def grad_out(layer: Layer, M: Optional[int] = None) -> Bf16Tensor:
    M = layer.M if M is None else M
    return bf16_normal((M, layer.N), 1.0, seed_of(layer.workload_id, "G"))


def small_layer(N: int, K: int, M: int, r: int, alpha: float, seed: int,
                name: str = "small") -> Layer:
    """A Layer with arbitrary (test) sizes; seed plays the workload id."""
    return Layer(name, seed, N, K, M, r, alpha)
