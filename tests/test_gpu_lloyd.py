"""GPU parity of the weighted Lloyd-Max learner (LowRA, section 5, mapping
and threshold learner) against the oracle.

Both sides run the learner in float64 from the same float32 data; they differ
only in the order in which an interval's sums are added (the oracle adds in
element order, the GPU from sorted 16-element segments in a fixed tree), so
every decision (assignment of a float32 x against a float64 threshold, the
stop test) comes out the same unless a value lies within a few float64 ulps
of a threshold or two errors tie that closely. Bar:
  * the same iteration count on every row;
  * every level within one float32 ulp of the oracle's, and at least 99 % of
    the rows bit-equal;
  * the thresholds are exactly the rounded-down midpoints of the returned
    float32 levels, and the unused slots hold the last level / 3.0.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import lloyd, nf4, codebook

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


def check_tables(L, T, bits):
    for i, b in enumerate(bits):
        n = 1 << int(b)
        assert np.array_equal(T[i, :n - 1].view(np.uint32),
                              nf4.midpoint_thresholds(L[i, :n]).view(np.uint32)), i
        assert np.all(T[i, n - 1:] == 3.0), i
        assert np.all(L[i, n:] == L[i, n - 1]), i
        assert np.all(np.diff(L[i, :n]) > 0), i


def check_against_oracle(L, T, it, W, bits, max_iters=lloyd.MAX_ITERS):
    Lr, Tr, itr = lloyd.learn_codebooks(W, bits, max_iters=max_iters, return_iters=True)
    assert np.array_equal(it, itr), np.nonzero(it != itr)
    up = np.nextafter(Lr, np.float32(np.inf))
    dn = np.nextafter(Lr, np.float32(-np.inf))
    assert np.all((L == Lr) | (L == up) | (L == dn))
    assert np.mean(np.all(L == Lr, axis=1)) >= 0.99
    check_tables(L, T, bits)


def sigma_rows(rng, N, K):
    sig = 0.02 * np.exp(0.3 * rng.standard_normal(N))
    return (rng.standard_normal((N, K)) * sig[:, None]).astype(np.float32)


def test_lloyd_mixed_widths(lq, torch):
    rng = np.random.default_rng(11)
    N, K = 96, 384
    W = sigma_rows(rng, N, K)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    L, T, it = lq.lloyd_codebooks(dev(torch, W), dev(torch, bits))
    check_against_oracle(host(L), host(T), host(it), W, bits)


@pytest.mark.parametrize("K", [64, 4096, 4160, 11008, 16384])
def test_lloyd_row_lengths(lq, torch, K):
    """One workgroup size per range of K (256, 512, 1024 threads), padding
    from 64 up to the sorted length."""
    rng = np.random.default_rng(K)
    N = 8
    W = sigma_rows(rng, N, K)
    bits = np.array([1, 2, 3, 4, 4, 3, 2, 1], dtype=np.uint8)
    L, T, it = lq.lloyd_codebooks(dev(torch, W), dev(torch, bits))
    check_against_oracle(host(L), host(T), host(it), W, bits)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_lloyd_half_inputs(lq, torch, dtype):
    rng = np.random.default_rng(3)
    N, K = 32, 512
    W = sigma_rows(rng, N, K)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    Wt = dev(torch, W).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    W32 = host(Wt.float())
    L, T, it = lq.lloyd_codebooks(Wt, dev(torch, bits))
    check_against_oracle(host(L), host(T), host(it), W32, bits)


def test_lloyd_degenerate_rows(lq, torch):
    """All-zero row (every interval empty, the error is 0/0 and never stops
    the loop: the NormalFloat levels come back after the iteration limit);
    a row with an all-zero block (zero weights); a constant row; a row of
    three distinct values (empty intervals keep their levels); a row with
    ties at +-1 in every block."""
    rng = np.random.default_rng(5)
    K = 256
    rows = []
    rows.append(np.zeros(K, np.float32))
    r = (rng.standard_normal(K) * 0.02).astype(np.float32); r[64:128] = 0.0; rows.append(r)
    rows.append(np.full(K, 0.01, np.float32))
    rows.append((rng.integers(-1, 2, K) * 0.02).astype(np.float32))
    r = (rng.standard_normal(K) * 0.02).astype(np.float32)
    for b in range(K // 64):
        r[64 * b] = 0.05; r[64 * b + 1] = -0.05
    rows.append(r)
    W = np.stack(rows)
    N = W.shape[0]
    for bits_val in (1, 2, 3, 4):
        bits = np.full(N, bits_val, np.uint8)
        L, T, it = lq.lloyd_codebooks(dev(torch, W), dev(torch, bits))
        L, T, it = host(L), host(T), host(it)
        Lr, Tr, itr = lloyd.learn_codebooks(W, bits, return_iters=True)
        assert np.array_equal(it, itr)
        assert np.array_equal(L.view(np.uint32), Lr.view(np.uint32))
        assert np.array_equal(T.view(np.uint32), Tr.view(np.uint32))
        assert it[0] == lloyd.MAX_ITERS
        assert np.array_equal(L[0, :1 << bits_val], lloyd.init_levels(bits_val).astype(np.float32))


@pytest.mark.parametrize("max_iters", [1, 2, 5])
def test_lloyd_iteration_limit(lq, torch, max_iters):
    rng = np.random.default_rng(17)
    N, K = 24, 320
    W = sigma_rows(rng, N, K)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    L, T, it = lq.lloyd_codebooks(dev(torch, W), dev(torch, bits), max_iters=max_iters)
    assert np.all(host(it) <= max_iters)
    check_against_oracle(host(L), host(T), host(it), W, bits, max_iters=max_iters)


def test_lloyd_row_bits_clamped(lq, torch):
    """Widths outside 1..4 are clamped, as in the codebook quantizer."""
    rng = np.random.default_rng(19)
    W = sigma_rows(rng, 4, 128)
    L0, T0, i0 = lq.lloyd_codebooks(dev(torch, W), dev(torch, np.array([0, 9, 1, 4], np.uint8)))
    L1, T1, i1 = lq.lloyd_codebooks(dev(torch, W), dev(torch, np.array([1, 4, 1, 4], np.uint8)))
    assert np.array_equal(host(L0), host(L1)) and np.array_equal(host(T0), host(T1))
    assert np.array_equal(host(i0), host(i1))


def test_lloyd_repeatable(lq, torch):
    rng = np.random.default_rng(23)
    W = dev(torch, sigma_rows(rng, 64, 1024))
    bits = dev(torch, rng.integers(1, 5, 64).astype(np.uint8))
    a = [host(x) for x in lq.lloyd_codebooks(W, bits)]
    b = [host(x) for x in lq.lloyd_codebooks(W, bits)]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_lloyd_tables_drive_codebook_quantizer(lq, torch):
    """Learned tables feed the codebook quantizer: its codes are the nearest
    learned level of every x (ties to the lower level)."""
    rng = np.random.default_rng(29)
    N, K = 40, 256
    W = sigma_rows(rng, N, K)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    L, T, _ = lq.lloyd_codebooks(dev(torch, W), dev(torch, bits))
    codes, absmax, row_off = lq.quantize_codebook(dev(torch, W), dev(torch, bits), T)
    packed, c, code_ref = codebook.quantize(W, bits, host(T))
    assert np.array_equal(host(codes)[:packed.size], packed)
    x = nf4.normalise(W, c).reshape(N, K).astype(np.float64)
    Lh = host(L).astype(np.float64)
    for i in range(N):
        n = 1 << int(bits[i])
        d = np.abs(x[i][:, None] - Lh[i, :n][None, :])
        assert np.array_equal(code_ref[i], np.argmin(d, axis=1))
