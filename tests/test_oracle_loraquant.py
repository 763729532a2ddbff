"""Pins for the LoRAQuant-style adapter quantization of the oracle (LoRAQuant
page, method overview and key design)."""
import numpy as np

from oracle import loraquant, nf4


def constructed(seed, N=96, K=128, r=6):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((N, r)))
    V, _ = np.linalg.qr(rng.standard_normal((K, r)))
    s = np.sort(rng.uniform(0.2, 2.0, r))[::-1]
    Rm = rng.standard_normal((r, r)) + 3 * np.eye(r)      # any invertible mixing
    B = (U * np.sqrt(s)) @ Rm
    A = np.linalg.solve(Rm, np.sqrt(s)[:, None] * V.T)
    return B, A, U, V, s


def test_reparam_recovers_the_svd_split():
    """B A = U diag(s) V^T built with a mixing matrix between the factors:
    the reparameterization undoes the mixing -- B' A' = B A, sigma = s,
    B' = U sqrt(s) and A' = sqrt(s) V^T up to one sign per component, with
    B'^T B' = A' A'^T = diag(s)."""
    B, A, U, V, s = constructed(0)
    Bp, Ap, sig = loraquant.reparam(B, A)
    assert np.allclose(sig, s, rtol=1e-12)
    assert np.allclose(Bp @ Ap, B @ A, atol=1e-12)
    assert np.allclose(Bp.T @ Bp, np.diag(s), atol=1e-12)
    assert np.allclose(Ap @ Ap.T, np.diag(s), atol=1e-12)
    for i in range(len(s)):
        sgn = np.sign(Ap[i] @ V[:, i])
        assert np.allclose(Ap[i], sgn * np.sqrt(s[i]) * V[:, i], atol=1e-12)
        assert np.allclose(Bp[:, i], sgn * np.sqrt(s[i]) * U[:, i], atol=1e-12)


def test_sign_convention():
    B, A, *_ = constructed(1)
    Bp, Ap, _ = loraquant.reparam(B, A)
    for i in range(Ap.shape[0]):
        k = int(np.argmax(np.abs(Ap[i])))
        assert Ap[i, k] > 0
    Bn, An, _ = loraquant.reparam(-B, A)          # same adapter up to sign: factors flip consistently
    assert np.allclose(Bn @ An, -(B @ A), atol=1e-12)


def test_choose_h_by_hand():
    s = np.array([3.0, 2.0, 1.0])                  # energies 9, 4, 1 of 14
    assert loraquant.choose_h(s, 0.6) == 1
    assert loraquant.choose_h(s, 9 / 14) == 1
    assert loraquant.choose_h(s, 0.65) == 2
    assert loraquant.choose_h(s, 0.9) == 2
    assert loraquant.choose_h(s, 0.93) == 3
    assert loraquant.choose_h(s, 1.0) == 3
    assert loraquant.choose_h(s, 0.0) == 1
    assert loraquant.choose_h(np.zeros(4), 0.9) == 0


def test_components_use_their_learned_nearest_levels():
    """Each component vector's codes pick its nearest learned level (ties to
    the lower), and the learned 1-bit levels leave less error than the fixed
    {-1, +1} start would (the learner never raises a row's error)."""
    rng = np.random.default_rng(2)
    B = (rng.standard_normal((128, 8)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    out = loraquant.loraquant(B, A, bits_hi=3, bits_lo=1, h=3)
    bits = out["bits"]
    qa = out["q"]["A"]
    X = out["Ap"]
    c = nf4.block_absmax(X)
    x = nf4.normalise(X, c).reshape(X.shape).astype(np.float64)
    got = (out["A_deq"] / np.repeat(c, 64).reshape(X.shape)).astype(np.float64)   # level per element
    for i, b in enumerate(bits):
        n = 1 << int(b)
        lv = qa["levels"][i, :n].astype(np.float64)
        near = lv[np.argmin(np.abs(x[i][:, None] - lv[None, :]), axis=1)]
        assert np.allclose(got[i], near, rtol=2 ** -8, atol=0)       # bf16 of level * absmax
    # 1-bit rows: learned levels beat the {-1, +1} start
    for i in np.nonzero(bits == 1)[0]:
        lv = qa["levels"][i, :2].astype(np.float64)
        err_learned = np.sum((x[i] - lv[(x[i] > qa["thresholds"][i, 0]).astype(int)]) ** 2)
        err_start = np.sum((x[i] - np.where(x[i] > 0, 1.0, -1.0)) ** 2)
        assert err_learned < err_start


def test_more_bits_less_error_and_zero_adapter():
    rng = np.random.default_rng(3)
    B = (rng.standard_normal((128, 16)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    e1 = loraquant.loraquant(B, A, rho=0.5, bits_hi=4, bits_lo=1)["rel_error"]
    e2 = loraquant.loraquant(B, A, rho=0.5, bits_hi=4, bits_lo=2)["rel_error"]
    e4 = loraquant.loraquant(B, A, rho=0.5, bits_hi=4, bits_lo=4)["rel_error"]
    assert e4 < e2 < e1
    z = loraquant.loraquant(np.zeros((64, 4), np.float32), A[:4, :128].copy(), rho=0.9)
    assert z["h"] == 0 and z["rel_error"] == 0.0 and not np.any(z["Bp"]) and not np.any(z["Ap"])
