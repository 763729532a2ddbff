"""Pins of the oracle's NF4 table, quantizer, packing and dequant against
facts fixed by the QLoRA page and by mathematics (not against itself)."""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import nf4, bf16


def test_table_construction_invariants():
    # QLoRA page, Contribution 1: 8 negative + 9 positive quantiles with the
    # duplicate 0 removed -> 16 values, exact zero, scaled into [-1, 1].
    q = nf4.levels()
    assert q.dtype == np.float32 and q.size == 16
    assert np.all(np.diff(q) > 0), "strictly increasing, distinct"
    assert q[0] == -1.0 and q[15] == 1.0
    assert q[7] == 0.0 and not np.signbit(q[7])
    assert np.sum(q < 0) == 7 and np.sum(q > 0) == 8


def test_table_is_equal_mass_quantiles():
    # each half: Phi(q_j * Phi^-1(delta)) equally spaced from 1/2 to delta
    # (checked with the CDF, a different routine from the quantile function).
    d = nf4.DELTA
    s = norm.ppf(d)
    q = nf4.levels_f64()
    pos = norm.cdf(q[q >= 0] * s)
    neg = norm.cdf(-q[q <= 0][::-1] * s)
    assert np.allclose(np.diff(pos), (d - 0.5) / 8, atol=1e-12)
    assert np.allclose(np.diff(neg), (d - 0.5) / 7, atol=1e-12)
    # denser near zero: gaps grow away from 0 on both sides
    gaps = np.diff(q)
    assert np.all(np.diff(gaps[7:]) > 0) and np.all(np.diff(gaps[:7]) < 0)


def test_thresholds_are_round_down_midpoints_exact():
    q = nf4.levels()
    t = nf4.thresholds()
    for i in range(15):
        m = (Fraction(float(q[i])) + Fraction(float(q[i + 1]))) / 2
        ti = Fraction(float(t[i]))
        nxt = Fraction(float(np.nextafter(t[i], np.float32(np.inf))))
        assert ti <= m < nxt
        # t_i itself is at least as close to q_i as to q_{i+1}
        assert abs(ti - Fraction(float(q[i]))) <= abs(ti - Fraction(float(q[i + 1])))
        # its successor is strictly closer to q_{i+1}
        assert abs(nxt - Fraction(float(q[i + 1]))) < abs(nxt - Fraction(float(q[i])))


def _near_threshold_values(width=40):
    t = nf4.thresholds()
    out = []
    for ti in t:
        v = np.float32(ti)
        lo = v
        for _ in range(width):
            lo = np.nextafter(lo, np.float32(-np.inf))
        cur = lo
        for _ in range(2 * width + 1):
            out.append(cur)
            cur = np.nextafter(cur, np.float32(np.inf))
    q = nf4.levels()
    out += list(q) + [np.float32(-0.0), np.float32(1e-40), np.float32(-1e-40)]
    return np.array(out, dtype=np.float32)


def test_count_rule_equals_bruteforce_nearest_ties_low():
    rng = np.random.default_rng(7)
    x = np.concatenate([_near_threshold_values(),
                        rng.uniform(-1, 1, 3000).astype(np.float32)])
    assert np.array_equal(nf4.count_above(x, nf4.thresholds()), nf4.nearest_code_bruteforce(x))


def test_quantize_small_blocks_bruteforce():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    W[1, :64] = 0.0                      # all-zero block
    W[2, 5] = -W[2, :64].__abs__().max() * 3  # negative absmax
    W[3, :64] = np.float32(0.013)          # constant block
    packed, c = nf4.quantize(W)
    assert packed.size == W.size // 2 and c.size == W.size // 64
    codes = nf4.unpack_nibbles(packed)
    flat = W.reshape(-1, 64)
    for j in range(flat.shape[0]):
        cj = np.abs(flat[j]).max()
        assert c[j] == cj
        if cj == 0:
            assert np.all(codes[64 * j:64 * j + 64] == 7)
            continue
        x = (flat[j] / cj).astype(np.float32)
        assert np.array_equal(codes[64 * j:64 * j + 64], nf4.nearest_code_bruteforce(x))
        # the absmax element maps to exactly +-1 -> an end code
        assert np.any(np.isin(codes[64 * j:64 * j + 64], [0, 15]))


def test_zero_weights_get_code_7():
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, 0] = 0.5
    W[0, 1] = -0.0
    codes = nf4.unpack_nibbles(nf4.quantize(W)[0])
    assert codes[1] == 7 and codes[2] == 7 and codes[0] == 15


def test_packing_high_nibble_first():
    # hand-built: codes 0..15 then 15..0 -> bytes 0x01, 0x23, ..., 0xFE, ..., 0x10
    codes = np.array(list(range(16)) + list(range(15, -1, -1)), dtype=np.uint8)
    p = nf4.pack_nibbles(codes)
    assert p[0] == 0x01 and p[1] == 0x23 and p[7] == 0xEF and p[8] == 0xFE and p[15] == 0x10
    assert np.array_equal(nf4.unpack_nibbles(p), codes)


def test_roundtrip_error_bound():
    # dequant(quant(w)) is within half of the largest level gap times absmax
    # (plus the float32 product and bfloat16 rounding).
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    packed, c = nf4.quantize(W)
    Wd = nf4.dequant(packed, c, W.shape)
    gap = np.max(np.diff(nf4.levels().astype(np.float64)))
    cb = np.repeat(c, 64).reshape(W.shape).astype(np.float64)
    err = np.abs(W.astype(np.float64) - Wd)
    assert np.all(err <= cb * gap / 2 + np.abs(Wd) * 2.0 ** -8 + cb * 2.0 ** -22)
    # and the element-wise error respects the local gap of its code
    codes = nf4.unpack_nibbles(packed).reshape(W.shape)
    q = nf4.levels().astype(np.float64)
    local = np.maximum(np.diff(np.r_[q[0], q])[codes], np.diff(np.r_[q, q[-1]])[codes])
    assert np.all(err <= cb * local / 2 + np.abs(Wd) * 2.0 ** -8 + cb * 2.0 ** -22)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1e-40, -3e-39,
                  3.0e38, 0.0, -0.0], dtype=np.float32),
        (rng.integers(0, 2 ** 16, 4000).astype(np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.f32_to_bf16_bits(x), want)


def test_fma_f32_is_single_rounding():
    rng = np.random.default_rng(9)
    a = rng.standard_normal(3000).astype(np.float32)
    b = (rng.standard_normal(3000) * 1e-3).astype(np.float32)
    c = rng.standard_normal(3000).astype(np.float32)
    # adversarial: a*b just off a float32 tie of c
    c[:100] = np.float32(1.0)
    a[:100] = np.float32(2.0 ** -24)
    b[:100] = (1.0 + rng.integers(-3, 4, 100) * 2.0 ** -23).astype(np.float32)
    got = bf16.fma_f32(a, b, c)
    for i in range(a.size):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        g = Fraction(float(got[i]))
        lo = Fraction(float(np.nextafter(got[i], np.float32(-np.inf))))
        hi = Fraction(float(np.nextafter(got[i], np.float32(np.inf))))
        # nearest float32: no neighbour is strictly closer; ties go to even
        assert abs(g - exact) <= abs(lo - exact) and abs(g - exact) <= abs(hi - exact)
        if abs(g - exact) == abs(lo - exact) or abs(g - exact) == abs(hi - exact):
            assert (np.float32(got[i]).view(np.uint32) & 1) == 0


def test_aqlora_error_of_exact_levels_is_zero():
    # AQLoRA page, section 3.1: a block made only of (absmax-scaled) NF4
    # levels round-trips exactly, so its error eps is 0.
    q = nf4.levels()
    W = np.tile(q * np.float32(0.5), 4).reshape(1, 64).astype(np.float32)
    assert nf4.roundtrip_error(W) == 0.0


def test_profile_error_matches_bruteforce_nearest():
    """eps from the threshold-count quantizer equals the error of a brute-force
    nearest-level reconstruction (independent code path, ties never hit by
    random data)."""
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    blocks = W.reshape(-1, 64)
    c = np.abs(blocks).max(axis=1)
    q = nf4.levels()
    total = 0.0
    for b, cb in zip(blocks, c):
        x = (b / cb).astype(np.float32)
        k = nf4.nearest_code_bruteforce(x, q)
        rec = (q[k] * cb).astype(np.float32).astype(np.float64)
        total += float(np.sum((b.astype(np.float64) - rec) ** 2))
    eps, s = nf4.profile(W)
    assert eps == pytest.approx(total / W.size, rel=1e-12)


def test_profile_power_of_two_scaling_is_exact():
    """Every step of the round trip commutes with a power-of-two scale, so
    eps(2^k W) = 4^k eps(W) exactly (no subnormals involved)."""
    rng = np.random.default_rng(22)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    e1, _ = nf4.profile(W)
    e2, _ = nf4.profile((W * np.float32(8.0)).astype(np.float32))
    assert e2 == 64.0 * e1


def test_profile_small_fraction_threshold():
    """s counts |w| < 0.01: the float32 nearest 0.01 lies just below it and
    counts; the next float32 up does not; signs do not matter."""
    t32 = np.float32(0.01)
    assert float(t32) < 0.01
    up = np.nextafter(t32, np.float32(1.0))
    W = np.array([t32, -t32, up, -up, 0.0, -0.0, 0.005, 0.5] + [1.0] * 56, dtype=np.float32).reshape(1, 64)
    _, s = nf4.profile(W)
    assert s == 5 / 64      # +-t32, +-0, 0.005


def test_profile_single_spike_blocks_have_zero_error():
    """A block with one nonzero weight maps it to +-1 (exact) and the zeros to
    the zero level, so its round trip is exact."""
    W = np.zeros((2, 64), dtype=np.float32)
    W[0, 5] = 0.037
    W[1, 60] = -3.5
    eps, s = nf4.profile(W)
    assert eps == 0.0
    assert s == 126 / 128
