"""The QLoRA layer, forward and backward, in float64.

QLoRA page, introduction: the frozen base weight is stored in 4 bits and
dequantized to BFloat16 when used, and the layer computes
    h = dequant(W0_NF4) x + (alpha / r) B A x,
where only A and B are updated by the optimizer (gradients flow through the
frozen 4-bit base to the adapter).

Row-vector convention (PyTorch Linear): X [M, K] holds M tokens, W' [N, K],
A [r, K], B [N, r], H [M, N]:
    t = X A^T                      [M, r]
    H = X W'^T + s t B^T,  s = alpha / r.
With L a scalar loss and G = dL/dH [M, N], the chain rule gives
    u = G B                        [M, r]
    dL/dB = s G^T t                [N, r]
    dL/dX = G W' + s u A           [M, K]
    dL/dA = s u^T X                [r, K]
and no gradient for the frozen W'. All products are float64 matmuls of the
exact bfloat16 / float32 input values.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(Wd, X, A, B, alpha: float, r: int = None):
    """Returns (H float64 [M, N], t float64 [M, r])."""
    Wd, X, A, B = _f64(Wd), _f64(X), _f64(A), _f64(B)
    r = A.shape[0] if r is None else r
    s = alpha / r
    t = X @ A.T
    H = X @ Wd.T + s * (t @ B.T)
    return H, t


def backward(Wd, X, G, A, B, alpha: float, r: int = None):
    """Returns (dX [M, K], dA [r, K], dB [N, r]) in float64."""
    Wd, X, G, A, B = _f64(Wd), _f64(X), _f64(G), _f64(A), _f64(B)
    r = A.shape[0] if r is None else r
    s = alpha / r
    t = X @ A.T
    u = G @ B
    dB = s * (G.T @ t)
    dX = G @ Wd + s * (u @ A)
    dA = s * (u.T @ X)
    return dX, dA, dB


def lora_down(X, A):
    """t = X A^T (float64)."""
    return _f64(X) @ _f64(A).T


def rel_frobenius(got, ref) -> float:
    got, ref = _f64(got), _f64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))
