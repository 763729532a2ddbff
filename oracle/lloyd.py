"""Weighted Lloyd-Max learner for per-channel mappings and thresholds.

LowRA page, section 5 (mapping and threshold learner):
  * each output channel's mapping (levels) and thresholds minimise that
    channel's mean squared error, posed as a weighted Lloyd-Max problem;
  * the weight of every element is the absmax of its 64-element block, so
    blocks with larger absmax count more;
  * thresholds start from the NormalFloat thresholds at 2 and 4 bits and
    from 0.0 at 1 bit;
  * each iteration recomputes the mapping as the weighted centroid of the
    data assigned to each code, then the thresholds as midpoints of adjacent
    levels; it stops at the iteration limit or when the MSE stops decreasing,
    and outputs the last computed mapping and thresholds.

Readings where the pages are silent:
  * data = the block-normalised values x = w / c (float32), weight = c;
  * 3 bits (not on the page) start from NF3, built like NF4 with 4 + 5 - 1
    levels; NF2 uses 2 + 3 - 1; the truncation probability of NF_b is
    1 - (1/(2*2^b) + 1/(2*(2^b - 1)))/2, which is NF4's for b = 4;
  * a bin that receives no data keeps its previous level; the levels before
    the first iteration are the NF_b levels ({-1, +1} at 1 bit);
  * the per-channel "average all thresholds" remark of the page is not
    applied, since it would undo per-channel thresholds;
  * the learner runs in float64; the output levels are rounded to float32 and
    the output thresholds are the float32 midpoints of those levels rounded
    toward -inf, so that quantizing with them maps x to its nearest level
    (ties low).
"""
from __future__ import annotations

import numpy as np

from .nf4 import levels_f64, block_absmax, normalise, midpoint_thresholds

MAX_ITERS = 100


def nf_delta(bits: int) -> float:
    n = 1 << bits
    return 1.0 - 0.5 * (1.0 / (2 * n) + 1.0 / (2 * (n - 1)))


def init_levels(bits: int) -> np.ndarray:
    if bits == 1:
        return np.array([-1.0, 1.0])
    return levels_f64(nf_delta(bits), half=1 << (bits - 1))


def init_thresholds(bits: int) -> np.ndarray:
    if bits == 1:
        return np.array([0.0])
    L = init_levels(bits)
    return (L[:-1] + L[1:]) / 2.0


def assign(x: np.ndarray, T: np.ndarray) -> np.ndarray:
    """x [R, K], T [R, n-1] -> code [R, K] = #thresholds strictly below x."""
    code = np.zeros(x.shape, dtype=np.int64)
    for k in range(T.shape[1]):
        code += x > T[:, k:k + 1]
    return code


def centroids(x, w, code, L_prev):
    """Weighted centroid of each bin; an empty bin keeps L_prev."""
    R, n = L_prev.shape
    idx = code + (np.arange(R)[:, None] * n)
    num = np.bincount(idx.ravel(), weights=(w * x).ravel(), minlength=R * n).reshape(R, n)
    den = np.bincount(idx.ravel(), weights=w.ravel(), minlength=R * n).reshape(R, n)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), L_prev)


def weighted_mse(x, w, code, L):
    rec = np.take_along_axis(L, code, axis=1)
    with np.errstate(invalid="ignore"):   # a row of zero weights gives 0/0 = NaN
        return np.sum(w * (x - rec) ** 2, axis=1) / np.sum(w, axis=1)


def lloyd_step(x, w, T, L_prev):
    """One iteration: assign by T, centroids, MSE of that assignment with the
    new levels, midpoints. Returns (L, T_next, mse)."""
    code = assign(x, T)
    L = centroids(x, w, code, L_prev)
    mse = weighted_mse(x, w, code, L)
    T_next = (L[:, :-1] + L[:, 1:]) / 2.0
    return L, T_next, mse


def learn(x, w, bits: int, max_iters: int = MAX_ITERS, history: list = None):
    """Weighted Lloyd-Max for R channels at once, each stopping on its own.
    x, w: [R, K] float64. Returns (L [R, 2^b] float64, T [R, 2^b - 1] float64,
    iterations [R])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    R = x.shape[0]
    T = np.tile(init_thresholds(bits), (R, 1))
    L = np.tile(init_levels(bits), (R, 1))
    prev = np.full(R, np.inf)
    active = np.ones(R, dtype=bool)
    iters = np.zeros(R, dtype=np.int64)
    for _ in range(max_iters):
        if not active.any():
            break
        a = np.nonzero(active)[0]
        La, Ta, mse = lloyd_step(x[a], w[a], T[a], L[a])
        L[a], T[a] = La, Ta
        iters[a] += 1
        if history is not None:
            history.append((a.copy(), mse.copy()))
        stop = mse >= prev[a]
        prev[a] = np.where(stop, prev[a], mse)
        active[a[stop]] = False
    return L, T, iters


def learn_codebooks(W: np.ndarray, row_bits: np.ndarray, block: int = 64,
                    max_iters: int = MAX_ITERS, return_iters: bool = False):
    """Per-row codebooks for W [N, K]. Returns (levels float32 [N, 16],
    thresholds float32 [N, 15]), plus the iterations computed per row when
    return_iters is set. A row with b bits uses the first 2^b levels and
    2^b - 1 thresholds; the unused level slots repeat the last level and the
    unused threshold slots hold 3.0 (above every normalised value)."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    c = block_absmax(W, block)
    x = normalise(W, c, block).reshape(N, K).astype(np.float64)
    wgt = np.repeat(c.astype(np.float64), block).reshape(N, K)
    levels = np.zeros((N, 16), dtype=np.float32)
    thresh = np.full((N, 15), 3.0, dtype=np.float32)
    iters = np.zeros(N, dtype=np.int64)
    row_bits = np.asarray(row_bits)
    for b in np.unique(row_bits):
        b = int(b)
        rows = np.nonzero(row_bits == b)[0]
        L, _, it = learn(x[rows], wgt[rows], b, max_iters)
        iters[rows] = it
        L32 = L.astype(np.float32)
        n = 1 << b
        levels[rows, :n] = L32
        levels[rows, n:] = L32[:, -1:]
        for j, i in enumerate(rows):
            thresh[i, :n - 1] = midpoint_thresholds(L32[j])
    if return_iters:
        return levels, thresh, iters
    return levels, thresh
