"""Pins of the oracle's QLoRA layer (QLoRA page, introduction): finite
differences for the backward, special cases with closed forms for the
forward, and shapes chosen so that a transposed operand cannot go unseen."""
import numpy as np

from oracle import layer


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(0)
    M, N, K, r, alpha = 3, 5, 7, 2, 6.0
    Wd, X, A, B, G = (_rand(rng, N, K), _rand(rng, M, K), _rand(rng, r, K),
                      _rand(rng, N, r), _rand(rng, M, N))

    def loss(X_, A_, B_):
        H, _ = layer.forward(Wd, X_, A_, B_, alpha)
        return float(np.sum(G * H))

    dX, dA, dB = layer.backward(Wd, X, G, A, B, alpha)
    h = 1e-6
    for P, grad, which in ((X, dX, 0), (A, dA, 1), (B, dB, 2)):
        D = _rand(rng, *P.shape)
        args_p = [X, A, B]
        args_m = [X, A, B]
        args_p[which] = P + h * D
        args_m[which] = P - h * D
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - np.sum(grad * D)) <= 1e-8 * max(1.0, abs(fd))


def test_lora_scale_is_alpha_over_r():
    # A selects feature 0, B writes it to output 1: the LoRA term of H is
    # (alpha / r) * X[:, 0] in column 1 (with W' = 0).
    M, N, K, r, alpha = 4, 3, 64, 16, 32.0
    rng = np.random.default_rng(1)
    X = _rand(rng, M, K)
    A = np.zeros((r, K)); A[0, 0] = 1.0
    B = np.zeros((N, r)); B[1, 0] = 1.0
    H, t = layer.forward(np.zeros((N, K)), X, A, B, alpha)
    assert np.allclose(H[:, 1], 2.0 * X[:, 0], rtol=0, atol=0)
    assert np.all(H[:, [0, 2]] == 0)
    assert np.array_equal(t[:, 0], X[:, 0])


def test_unit_vector_probe_reads_weight_columns():
    # X rows = e_k and B = 0: H[m, n] = W'[n, k_m]
    N, K, r = 6, 10, 2
    rng = np.random.default_rng(2)
    Wd = _rand(rng, N, K)
    ks = [3, 0, 9]
    X = np.zeros((3, K)); X[np.arange(3), ks] = 1.0
    H, _ = layer.forward(Wd, X, _rand(rng, r, K), np.zeros((N, r)), 8.0)
    assert np.array_equal(H, Wd[:, ks].T)
    # G rows = e_n and B = 0: dX row = W'[n, :]
    G = np.zeros((2, N)); G[0, 4] = 1.0; G[1, 1] = 1.0
    dX, dA, dB = layer.backward(Wd, np.zeros((2, K)), G, _rand(rng, r, K), np.zeros((N, r)), 8.0)
    assert np.array_equal(dX, Wd[[4, 1]])
    assert np.all(dA == 0)


def test_merged_weight_identity():
    # H equals X (W' + s B A)^T: the adapter is a rank-r update of W'
    rng = np.random.default_rng(3)
    M, N, K, r, alpha = 5, 4, 9, 3, 12.0
    Wd, X, A, B = _rand(rng, N, K), _rand(rng, M, K), _rand(rng, r, K), _rand(rng, N, r)
    H, _ = layer.forward(Wd, X, A, B, alpha)
    merged = Wd + (alpha / r) * (B @ A)
    assert np.allclose(H, X @ merged.T, rtol=1e-12, atol=1e-12)


def test_rel_frobenius():
    a = np.ones((2, 2))
    assert layer.rel_frobenius(a, a) == 0.0
    assert abs(layer.rel_frobenius(a * 1.001, a) - 1e-3) < 1e-12
