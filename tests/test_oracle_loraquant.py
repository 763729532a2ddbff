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


def test_nf_tables():
    lv, th = loraquant.nf_tables(4)
    assert np.array_equal(lv, nf4.levels()) and np.array_equal(th, nf4.thresholds())
    lv, th = loraquant.nf_tables(1)
    assert np.array_equal(lv[:2], [-1.0, 1.0]) and np.all(lv[2:] == 1.0)
    assert th[0] == 0.0 and np.all(th[1:] == 3.0)


def test_four_bit_components_are_nf4_rows():
    """With 4 bits everywhere each component vector is NF4-quantized: the
    dequantized A' equals NF4's dequantization of A' with float32 constants."""
    rng = np.random.default_rng(2)
    B = (rng.standard_normal((128, 8)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    out = loraquant.loraquant(B, A, bits_hi=4, bits_lo=4, h=3)
    packed, c = nf4.quantize(out["Ap"])
    assert np.array_equal(out["A_deq"].astype(np.float32), nf4.dequant(packed, c, out["Ap"].shape))
    packed, c = nf4.quantize(np.ascontiguousarray(out["Bp"].T))
    assert np.array_equal(out["B_deq"].T.astype(np.float32), nf4.dequant(packed, c, (8, 128)))


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
