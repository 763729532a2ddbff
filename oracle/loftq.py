"""LoftQ-style initialisation of the low-rank adapter over an NF4 base.

LowRA page:
  * section 3 (workflow): after the base weight is quantized, the
    quantization error is computed and a low-rank initialiser turns it into
    the starting adapter, so that the adapter absorbs the error; LoftQ is the
    initialiser chosen;
  * section 5 (low-rank initialiser): quantizing first and taking the SVD of
    what quantization leaves lets the low-rank tensors absorb the error;
    following LoftQ, five alternating steps are run.

Reading of the alternation (the page names it, it does not spell it out),
for t = 1 .. steps, starting from B = 0, A = 0:
    Q_t     = NF4(W - B A)                 (quantize the weight minus the adapter)
    R_t     = W - dequant(Q_t)             (what the quantized base misses)
    B, A    = rank-r SVD of R_t            (the adapter that absorbs it)
The rank-r SVD is the truncated SVD R ~ U_r S_r V_r^T, split evenly:
B = U_r S_r^(1/2) [N, r], A = S_r^(1/2) V_r^T [r, K] (the page does not give
the split; an even split keeps both factors on the same scale).

Precision readings (shared with the GPU path by definition, not by code):
  * W - B A: the rank-r product is summed in float64 over j = 0 .. r-1 in
    that order from the float32 factors (each product exact in float64), and
    W - sum is rounded once to float32;
  * dequant is the layer's bfloat16 weight (with or without double
    quantization of the block constants); R = float32(W - W');
  * the factors are kept in float32 between steps.
"""
from __future__ import annotations

import numpy as np

from . import nf4, dq

STEPS = 5


def lowrank_sub(W: np.ndarray, B: np.ndarray, A: np.ndarray) -> np.ndarray:
    """float32(W - sum_j B[:, j] A[j, :]), the sum in float64 in order of j."""
    W = np.asarray(W, dtype=np.float32)
    B = np.asarray(B, dtype=np.float32).astype(np.float64)
    A = np.asarray(A, dtype=np.float32).astype(np.float64)
    acc = np.zeros(W.shape, dtype=np.float64)
    for j in range(B.shape[1]):
        acc += B[:, j:j + 1] * A[j:j + 1, :]
    return (W.astype(np.float64) - acc).astype(np.float32)


def quantize_dequant(Wt: np.ndarray, double_quant: bool):
    """NF4 quantization of Wt and the layer's bfloat16 view of it. Returns
    (packed codes, float32 absmax, DQ triple or None, W' as float32)."""
    packed, c = nf4.quantize(Wt)
    if double_quant:
        code8, s2, mu = dq.double_quant(c)
        cp = dq.dq_decode(code8, s2, mu)
        dqt = (code8, s2, mu)
    else:
        cp, dqt = c, None
    Wd = nf4.dequant(packed, cp, Wt.shape)
    return packed, c, dqt, Wd


def residual(W: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """R = float32(W - W') (one float32 subtraction per element)."""
    return (np.asarray(W, dtype=np.float32) - np.asarray(Wd, dtype=np.float32)).astype(np.float32)


def svd_rank(R: np.ndarray, r: int):
    """Truncated SVD of R in float64, split evenly: returns (B [N, r],
    A [r, K], sigma [r]) with B A the best rank-r approximation of R."""
    U, s, Vt = np.linalg.svd(np.asarray(R, dtype=np.float64), full_matrices=False)
    h = np.sqrt(s[:r])
    return U[:, :r] * h[None, :], h[:, None] * Vt[:r], s[:r]


def objective(W: np.ndarray, Wd: np.ndarray, B: np.ndarray, A: np.ndarray) -> float:
    """||W - W' - B A||_F^2 in float64."""
    E = np.asarray(W, np.float64) - np.asarray(Wd, np.float64) - np.asarray(B, np.float64) @ np.asarray(A, np.float64)
    return float(np.sum(E * E))


def loftq(W: np.ndarray, r: int, steps: int = STEPS, double_quant: bool = True, svd=svd_rank):
    """The alternation above. Returns a dict with the final packed codes,
    constants (float32 absmax and the DQ triple), float32 factors B [N, r],
    A [r, K], the last singular values, and per step the objective
    ||W - W'_t - B_t A_t||_F^2 (the error the adapter leaves)."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    B = np.zeros((N, r), np.float32)
    A = np.zeros((r, K), np.float32)
    objs = []
    out = {}
    for _ in range(steps):
        Wt = lowrank_sub(W, B, A)
        packed, c, dqt, Wd = quantize_dequant(Wt, double_quant)
        R = residual(W, Wd)
        B64, A64, s = svd_rank(R, r)
        B, A = B64.astype(np.float32), A64.astype(np.float32)
        objs.append(objective(W, Wd, B, A))
        out = {"packed": packed, "absmax": c, "dq": dqt, "Wd": Wd, "sigma": s}
    out.update({"B": B, "A": A, "objectives": np.array(objs)})
    return out
