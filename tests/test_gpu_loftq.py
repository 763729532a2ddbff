"""GPU parity of the LoftQ-style initialiser (LowRA, sections 3 and 5)
against the oracle.

  * W - B A and the residual W - W' are bit-exact (same float64 sum order,
    same single roundings).
  * The rank-r SVD is randomized subspace iteration on the GPU and the exact
    truncated SVD in the oracle. Where the top-r singular values are
    separated from the rest, the answer is unique and the GPU factors must
    match it (1e-5). On a quantization residual the spectrum is flat, so only
    what is unique is compared: the singular values (Ritz values never
    exceed them; within 3 % at 8 power steps, 0.5 % at 32) and the error left
    (within 2e-3 of the optimum at 8 steps), plus B^T B = A A^T = diag(sigma).
  * The alternation: the quantizations it performs are bit-exact given its
    own adapters, its reported objectives match the oracle's recomputation
    from its outputs, and its final error is within 1 % of the oracle's
    exact-SVD alternation.
"""
import numpy as np
import pytest

from oracle import loftq, nf4, dq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lq():
    import quantized_lora_fine_lq_amd as mod
    return mod


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def omega(K, l, seed=99):
    return np.random.default_rng(seed).standard_normal((K, l)).astype(np.float32)


def nf4_residual(W, double_quant=True):
    _, _, _, Wd = loftq.quantize_dequant(W, double_quant)
    return loftq.residual(W, Wd), Wd


@pytest.mark.parametrize("N,K,r", [(64, 256, 0), (64, 256, 1), (200, 512, 16), (96, 1024, 64)])
def test_lowrank_sub_bit_exact(lq, torch, N, K, r):
    rng = np.random.default_rng(N + K + r)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.01).astype(np.float32)
    A = (rng.standard_normal((r, K)) * 0.01).astype(np.float32)
    out = host(lq.lowrank_sub(dev(torch, W), dev(torch, B), dev(torch, A)))
    ref = loftq.lowrank_sub(W, B, A)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_residual_bit_exact(lq, torch):
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((128, 512)) * 0.02).astype(np.float32)
    qw = lq.QWeight.from_weight(dev(torch, W))
    Wd = lq.dequant(qw)
    R = host(lq.residual(dev(torch, W), Wd))
    Rref, _ = nf4_residual(W, True)
    assert np.array_equal(R.view(np.uint32), Rref.view(np.uint32))


def check_factor_shape(B, A, sigma, tol):
    assert np.all(np.diff(sigma) <= 0)
    assert np.allclose(B.T.astype(np.float64) @ B, np.diag(sigma), atol=tol * sigma[0])
    assert np.allclose(A.astype(np.float64) @ A.T, np.diag(sigma), atol=tol * sigma[0])


@pytest.mark.parametrize("N,K,r,l,q", [(192, 256, 8, 16, 2), (300, 200, 16, 32, 4), (512, 384, 40, 64, 4)])
def test_svd_unique_case_matches(lq, torch, N, K, r, l, q):
    """Rank-r signal with separated singular values plus small noise: the
    truncated SVD is unique and the GPU factors must reproduce it."""
    rng = np.random.default_rng(N + r)
    U, _ = np.linalg.qr(rng.standard_normal((N, r)))
    V, _ = np.linalg.qr(rng.standard_normal((K, r)))
    R = ((U * np.linspace(10.0, 4.0, r)) @ V.T + 1e-3 * rng.standard_normal((N, K))).astype(np.float32)
    B, A, s = (host(x) for x in lq.svd_lowrank(dev(torch, R), r, dev(torch, omega(K, l)), power_iters=q))
    Bo, Ao, so = loftq.svd_rank(R, r)
    assert np.max(np.abs(s - so) / so) <= 1e-5
    ref = Bo @ Ao
    assert np.linalg.norm(B.astype(np.float64) @ A - ref) <= 1e-5 * np.linalg.norm(ref)
    check_factor_shape(B, A, s, 1e-5)


@pytest.mark.parametrize("q,sig_tol,obj_tol", [(8, 0.03, 2e-3), (32, 0.005, 2e-4)])
def test_svd_on_quantization_residual(lq, torch, q, sig_tol, obj_tol):
    rng = np.random.default_rng(3)
    N, K, r, l = 256, 512, 16, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    R, _ = nf4_residual(W)
    B, A, s = (host(x) for x in lq.svd_lowrank(dev(torch, R), r, dev(torch, omega(K, l)), power_iters=q))
    Bo, Ao, so = loftq.svd_rank(R, r)
    assert np.all(s <= so * (1 + 1e-5))
    assert np.all(s >= so * (1 - sig_tol))
    E = R - B.astype(np.float64) @ A
    Eo = R - Bo @ Ao
    opt = np.sum(Eo * Eo)
    assert opt <= np.sum(E * E) <= opt * (1 + obj_tol)
    check_factor_shape(B, A, s, 1e-5)


def test_svd_zero_and_rank_deficient(lq, torch):
    """A zero matrix gives zero factors; a rank-3 matrix gives three
    components and zero factors past its rank."""
    N, K, r, l = 128, 256, 8, 16
    B, A, s = (host(x) for x in lq.svd_lowrank(dev(torch, np.zeros((N, K), np.float32)), r,
                                               dev(torch, omega(K, l)), power_iters=2))
    assert np.all(B == 0) and np.all(A == 0) and np.all(s == 0)
    rng = np.random.default_rng(4)
    R = (rng.standard_normal((N, 3)) @ rng.standard_normal((3, K))).astype(np.float32)
    B, A, s = (host(x) for x in lq.svd_lowrank(dev(torch, R), r, dev(torch, omega(K, l)), power_iters=2))
    so = np.linalg.svd(R.astype(np.float64), compute_uv=False)
    assert np.allclose(s[:3], so[:3], rtol=1e-5)
    assert np.all(s[3:] <= 1e-4 * so[0])
    assert np.linalg.norm(B.astype(np.float64) @ A - R) <= 1e-5 * np.linalg.norm(R)


def test_svd_repeatable(lq, torch):
    rng = np.random.default_rng(5)
    R = dev(torch, (rng.standard_normal((256, 320)) * 0.01).astype(np.float32))
    Om = dev(torch, omega(320, 32))
    a = [host(x) for x in lq.svd_lowrank(R, 16, Om)]
    b = [host(x) for x in lq.svd_lowrank(R, 16, Om)]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def oracle_view(lq, qw, double_quant):
    """The GPU's quantized weight as the oracle decodes it (bf16 W')."""
    packed = host(qw.codes)
    if double_quant:
        cp = dq.dq_decode(host(qw.absmax_q), host(qw.dq_scale), host(qw.dq_mean)[0])
    else:
        cp = host(qw.absmax)
    return packed, cp


@pytest.mark.parametrize("double_quant", [True, False])
def test_loftq_steps_and_objectives(lq, torch, double_quant):
    """Step 1 is plain NF4 of W; step 2 quantizes W - B1 A1 with the GPU's
    own step-1 factors; the reported objective equals the oracle's
    recomputation from the returned codes and factors."""
    rng = np.random.default_rng(6)
    N, K, r, l = 192, 512, 16, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wd_, Om = dev(torch, W), dev(torch, omega(K, l))
    qw1, B1, A1, s1, obj1 = lq.loftq_init(Wd_, r, Om, steps=1, double_quant=double_quant)
    packed, c = nf4.quantize(W)
    assert np.array_equal(host(qw1.codes), packed) and np.array_equal(host(qw1.absmax_f32), c)
    if double_quant:
        code8, s2, mu = dq.double_quant(c)
        assert np.array_equal(host(qw1.absmax_q), code8) and host(qw1.dq_mean)[0] == mu
    qw2, B2, A2, s2_, obj2 = lq.loftq_init(Wd_, r, Om, steps=2, double_quant=double_quant)
    packed2, c2 = nf4.quantize(loftq.lowrank_sub(W, host(B1), host(A1)))
    assert np.array_equal(host(qw2.codes), packed2) and np.array_equal(host(qw2.absmax_f32), c2)
    o2 = host(obj2)
    assert host(obj1)[0] == o2[0]
    pk, cp = oracle_view(lq, qw2, double_quant)
    Rr = loftq.residual(W, nf4.dequant(pk, cp, W.shape)).astype(np.float64)
    E = Rr - host(B2).astype(np.float64) @ host(A2).astype(np.float64)
    ref = float(np.sum(E * E))
    assert abs(o2[1] - ref) <= 1e-9 * ref


def test_loftq_close_to_exact_alternation(lq, torch):
    """Five steps: the error left is below plain NF4's and within 1 % of the
    oracle's exact-SVD alternation."""
    rng = np.random.default_rng(7)
    N, K, r, l = 256, 512, 16, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qw, B, A, s, obj = lq.loftq_init(dev(torch, W), r, dev(torch, omega(K, l)), steps=5, power_iters=16)
    ref = loftq.loftq(W, r, steps=5, double_quant=True)
    R, _ = nf4_residual(W)
    plain = float(np.sum(R.astype(np.float64) ** 2))
    got = host(obj)[-1]
    assert got < plain
    assert got <= ref["objectives"][-1] * 1.01
