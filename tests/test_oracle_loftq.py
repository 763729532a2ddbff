"""Pins for the LoftQ-style initialiser of the oracle (LowRA page, sections 3
and 5): each step checked against values fixed by construction."""
from fractions import Fraction

import numpy as np

from oracle import loftq, nf4


def test_lowrank_sub_zero_adapter_is_identity():
    rng = np.random.default_rng(0)
    W = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    out = loftq.lowrank_sub(W, np.zeros((8, 3), np.float32), np.zeros((3, 128), np.float32))
    assert np.array_equal(out.view(np.uint32), W.view(np.uint32))


def test_lowrank_sub_exact_small_integers():
    """Factors and weights on a coarse dyadic grid: every product and sum is
    exact, so the result must be the exact W - B A (orientation, sign and
    indices of the product)."""
    rng = np.random.default_rng(1)
    N, K, r = 5, 7, 3
    B = (rng.integers(-8, 9, (N, r)) / 4).astype(np.float32)
    A = (rng.integers(-8, 9, (r, K)) / 8).astype(np.float32)
    W = (rng.integers(-64, 65, (N, K)) / 16).astype(np.float32)
    out = loftq.lowrank_sub(W, B, A)
    for n in range(N):
        for k in range(K):
            exact = Fraction(float(W[n, k])) - sum(Fraction(float(B[n, j])) * Fraction(float(A[j, k]))
                                                   for j in range(r))
            assert Fraction(float(out[n, k])) == exact


def random_orthogonal(rng, n, m):
    Q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return Q


def test_svd_rank_recovers_constructed_spectrum():
    """R = U diag(s) V^T with known orthonormal U, V and distinct s: the
    rank-r factors rebuild the top-r part, sigma is s[:r], B's columns are
    orthogonal with squared norms s, and the error left is sum_{i>r} s_i^2
    (Eckart-Young)."""
    rng = np.random.default_rng(2)
    N, K, m, r = 40, 30, 12, 5
    U = random_orthogonal(rng, N, m)
    V = random_orthogonal(rng, K, m)
    s = np.sort(rng.uniform(0.5, 3.0, m))[::-1]
    R = (U * s) @ V.T
    B, A, sig = loftq.svd_rank(R, r)
    assert np.allclose(sig, s[:r], rtol=1e-12, atol=0)
    top = (U[:, :r] * s[:r]) @ V[:, :r].T
    assert np.allclose(B @ A, top, rtol=0, atol=1e-12)
    G = B.T @ B
    assert np.allclose(G, np.diag(s[:r]), atol=1e-12)
    E = R - B @ A
    assert abs(np.sum(E * E) - np.sum(s[r:] ** 2)) <= 1e-10 * np.sum(s ** 2)


def test_residual_vanishes_on_the_grid():
    """Blocks whose values are bfloat16 roundings of NF4 levels, each block
    holding -1 and +1 (absmax 1): dequantization gives the weights back, so
    the residual is exactly zero."""
    rng = np.random.default_rng(3)
    q = nf4.levels()
    qb = nf4.round_bf16(q)
    W = qb[rng.integers(0, 16, (4, 256))].astype(np.float32)
    W[:, ::64] = -1.0
    W[:, 1::64] = 1.0
    packed, c, dqt, Wd = loftq.quantize_dequant(W, double_quant=False)
    assert np.all(c == 1.0)
    R = loftq.residual(W, Wd)
    assert np.all(R == 0.0)


def test_full_rank_adapter_absorbs_everything():
    """r = min(N, K): the adapter can represent any residual, so after one
    step only the float32 rounding of the factors is left."""
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((24, 64)) * 0.02).astype(np.float32)
    out = loftq.loftq(W, r=24, steps=1, double_quant=True)
    R = loftq.residual(W, out["Wd"])
    assert out["objectives"][0] <= 1e-10 * float(np.sum(R.astype(np.float64) ** 2))


def test_adapter_removes_the_top_singular_energy():
    """Step 1: the error left equals ||R||^2 minus the energy of the r
    largest singular values of R, which is below the plain quantization
    error ||R||^2 (the rank-0 case)."""
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((64, 192)) * 0.02).astype(np.float32)
    out = loftq.loftq(W, r=8, steps=1, double_quant=False)
    R = loftq.residual(W, out["Wd"]).astype(np.float64)
    plain = float(np.sum(R * R))
    left = plain - float(np.sum(out["sigma"] ** 2))
    assert abs(out["objectives"][0] - left) <= 1e-6 * plain
    assert out["objectives"][0] < plain
    zero = loftq.loftq(W, r=0, steps=1, double_quant=False)
    assert abs(zero["objectives"][0] - plain) <= 1e-12 * plain


def test_first_quantization_is_plain_nf4():
    """Step 1 quantizes W itself (the adapter starts at zero)."""
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    out = loftq.loftq(W, r=4, steps=1, double_quant=False)
    packed, c = nf4.quantize(W)
    assert np.array_equal(out["packed"], packed) and np.array_equal(out["absmax"], c)


def test_second_step_quantizes_weight_minus_first_adapter():
    """Step t quantizes W - B_{t-1} A_{t-1} with the previous step's float32
    factors, and its adapter comes from the new residual."""
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((32, 128)) * 0.02).astype(np.float32)
    one = loftq.loftq(W, r=4, steps=1, double_quant=True)
    two = loftq.loftq(W, r=4, steps=2, double_quant=True)
    packed, c = nf4.quantize(loftq.lowrank_sub(W, one["B"], one["A"]))
    assert np.array_equal(two["packed"], packed) and np.array_equal(two["absmax"], c)
    assert not np.array_equal(two["packed"], one["packed"])
    B2, A2, _ = loftq.svd_rank(loftq.residual(W, two["Wd"]), 4)
    assert np.allclose(two["B"] @ two["A"], B2 @ A2, atol=1e-6)
