"""LoRAQuant-style mixed-precision quantization of a LoRA adapter.

LoRAQuant page ("LoRAQuant: Mixed-Precision Quantization of LoRA to Ultra-Low
Bits"), method overview and key design:
  * the adapter B A is reparameterized by its SVD, so that the important
    information sits in a few rows (of A) and columns (of B);
  * which components are important is decided from the singular values;
  * the important components are quantized at a higher precision, the rest
    at an ultra-low bit width; the quantized adapter is then used as usual.

Readings where the page is silent:
  * the SVD is split evenly: with B A = U S V^T (rank r),
    B' = U S^(1/2) [N, r], A' = S^(1/2) V^T [r, K]; component i is column i of
    B' and row i of A';
  * sign of a component: the entry of largest magnitude in row i of A' is
    positive (the first such entry on ties), column i of B' flips with it;
  * importance: the h largest components, h the smallest count whose squared
    singular values reach a fraction rho of the total (at least 1 when the
    adapter is nonzero), unless h is given;
  * quantizer: each component vector (row of A', column of B') is a
    codebook row of this framework: 64-element groups scaled by their absmax,
    codes = number of thresholds below x, with its own levels and thresholds
    learned by the weighted Lloyd-Max learner at its width (started from the
    NormalFloat tables of that width); b_hi bits for the h important
    components, b_lo bits for the rest. (With fixed NormalFloat tables a
    1-bit vector would become +-absmax everywhere, about 2.5 times its RMS for
    Gaussian-like data; the learned 1-bit levels sit near the mean |x|.)
  * arithmetic: the reparameterized factors are formed in float64 and stored
    as float32, which is what gets quantized.
"""
from __future__ import annotations

import numpy as np

from . import codebook, lloyd


def reparam(B: np.ndarray, A: np.ndarray):
    """(B' [N, r] float64, A' [r, K] float64, sigma [r]) from the SVD of B A."""
    B = np.asarray(B, np.float64)
    A = np.asarray(A, np.float64)
    r = B.shape[1]
    U, s, Vt = np.linalg.svd(B @ A, full_matrices=False)
    U, s, Vt = U[:, :r], s[:r], Vt[:r]
    h = np.sqrt(s)
    Bp = U * h[None, :]
    Ap = h[:, None] * Vt
    for i in range(r):
        k = int(np.argmax(np.abs(Ap[i])))
        if Ap[i, k] < 0:
            Ap[i] = -Ap[i]
            Bp[:, i] = -Bp[:, i]
    return Bp, Ap, s


def choose_h(sigma: np.ndarray, rho: float) -> int:
    """Smallest h with sum_{i<h} sigma_i^2 >= rho * sum sigma_i^2 (0 for a
    zero adapter)."""
    e = np.asarray(sigma, np.float64) ** 2
    c = np.cumsum(e)            # in order; the total is its last entry
    tot = float(c[-1]) if len(c) else 0.0
    if tot == 0.0:
        return 0
    return int(min(len(e), max(1, int(np.searchsorted(c, rho * tot, side="left")) + 1)))


def component_bits(r: int, h: int, bits_hi: int, bits_lo: int) -> np.ndarray:
    return np.array([bits_hi if i < h else bits_lo for i in range(r)], np.uint8)


def quantize(Bp32: np.ndarray, Ap32: np.ndarray, bits: np.ndarray):
    """Per-component learned codebooks for A' rows and B'^T rows, then their
    codebook quantization. Returns dicts for A and B: packed, absmax,
    offsets, levels [r, 16], thresholds [r, 15], shape."""
    out = {}
    for name, X in (("A", np.asarray(Ap32, np.float32)), ("B", np.ascontiguousarray(np.asarray(Bp32, np.float32).T))):
        lv, th = lloyd.learn_codebooks(X, bits)
        packed, c, _ = codebook.quantize(X, bits, th)
        out[name] = {"packed": packed, "absmax": c, "offsets": codebook.row_offsets(bits, X.shape[1]),
                     "levels": lv, "thresholds": th, "shape": X.shape}
    return out


def dequant(q: dict, bits: np.ndarray) -> np.ndarray:
    """bfloat16 values (as float32) of a quantized A' or B'^T."""
    n, k = q["shape"]
    return codebook.dequant(q["packed"], bits, q["levels"], q["absmax"], n, k)


def loraquant(B: np.ndarray, A: np.ndarray, rho: float = 0.9, bits_hi: int = 3, bits_lo: int = 1, h: int = None):
    """The whole method: returns the float32 factors, sigma, h, bits, the
    quantized parts and the relative Frobenius error of the dequantized
    adapter against B A."""
    Bp, Ap, s = reparam(B, A)
    hh = choose_h(s, rho) if h is None else int(h)
    bits = component_bits(B.shape[1], hh, bits_hi, bits_lo)
    Bp32, Ap32 = Bp.astype(np.float32), Ap.astype(np.float32)
    q = quantize(Bp32, Ap32, bits)
    Ad = dequant(q["A"], bits).astype(np.float64)
    Bd = dequant(q["B"], bits).astype(np.float64).T
    ref = np.asarray(B, np.float64) @ np.asarray(A, np.float64)
    err = float(np.linalg.norm(Bd @ Ad - ref) / np.linalg.norm(ref)) if np.any(ref) else 0.0
    return {"Bp": Bp32, "Ap": Ap32, "sigma": s, "h": hh, "bits": bits, "q": q, "A_deq": Ad, "B_deq": Bd,
            "rel_error": err}
