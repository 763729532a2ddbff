"""Pins of the oracle's per-channel codebook quantizer (LowRA page, sections
3 and 4.1) and weighted Lloyd-Max learner (section 5)."""
import math

import numpy as np

from oracle import codebook, lloyd, nf4


def test_four_bit_with_nf4_tables_equals_nf4():
    rng = np.random.default_rng(0)
    N, K = 6, 192
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    T = np.tile(nf4.thresholds(), (N, 1))
    packed, c, codes = codebook.quantize(W, np.full(N, 4), T)
    p_nf4, c_nf4 = nf4.quantize(W)
    assert np.array_equal(c, c_nf4)
    assert np.array_equal(codes.reshape(-1), nf4.unpack_nibbles(p_nf4))
    L = np.tile(nf4.levels(), (N, 1))
    assert np.array_equal(codebook.dequant(packed, np.full(N, 4), L, c, N, K),
                          nf4.dequant(p_nf4, c, (N, K)))


def test_one_bit_threshold_zero_is_sign():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((3, 128))).astype(np.float32)
    W[0, 3] = 0.0
    T = np.full((3, 15), 3.0, dtype=np.float32); T[:, 0] = 0.0
    packed, c, codes = codebook.quantize(W, np.ones(3), T)
    assert np.array_equal(codes, (W > 0).astype(np.uint8))
    assert packed.size == 3 * 128 // 8


def test_bit_plane_layout_by_hand():
    # one 64-block at 3 bits: element e has code e % 8 -> plane p bit e = bit p of e
    codes = (np.arange(64) % 8).astype(np.uint8)
    b = codebook.pack_planes(codes, 3)
    assert b.size == 24
    words = b.view("<u8")
    for p in range(3):
        want = sum(1 << e for e in range(64) if (e % 8) >> p & 1)
        assert int(words[p]) == want
    assert np.array_equal(codebook.unpack_planes(b, 3, 64), codes)


def test_codes_bruteforce_with_random_thresholds():
    rng = np.random.default_rng(2)
    N, K = 8, 128
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bits = np.array([1, 2, 3, 4, 4, 3, 2, 1])
    T = np.full((N, 15), 3.0, dtype=np.float32)
    for i, b in enumerate(bits):
        T[i, :(1 << b) - 1] = np.sort(rng.uniform(-1, 1, (1 << b) - 1)).astype(np.float32)
    packed, c, codes = codebook.quantize(W, bits, T)
    off = codebook.row_offsets(bits, K)
    assert off[-1] == sum(K * b // 8 for b in bits)
    for i in range(N):
        for k in range(K):
            cj = c[(i * K + k) // 64]
            x = np.float32(W[i, k] / cj)
            # scan: the bin whose left edge is the last threshold below x
            code = 0
            for m in range((1 << bits[i]) - 1):
                if x > T[i, m]:
                    code = m + 1
            assert codes[i, k] == code
        assert np.array_equal(codebook.unpack_planes(packed[off[i]:off[i + 1]], bits[i], K), codes[i])


def _data(rng, R=4, K=512):
    x = np.clip(rng.standard_normal((R, K)) / 2.5, -1, 1)
    w = np.repeat(rng.uniform(0.5, 2.0, (R, K // 64)), 64, axis=1)
    return x, w


def test_lloyd_mse_non_increasing_and_stops():
    rng = np.random.default_rng(3)
    x, w = _data(rng)
    for b in (1, 2, 3, 4):
        hist = []
        L, T, it = lloyd.learn(x, w, b, history=hist)
        per_row = {i: [] for i in range(x.shape[0])}
        for rows, mse in hist:
            for i, m in zip(rows, mse):
                per_row[i].append(m)
        for i, ms in per_row.items():
            # every accepted step decreased the MSE; the last one did not
            assert all(ms[j + 1] < ms[j] for j in range(len(ms) - 2))
            assert len(ms) == lloyd.MAX_ITERS or ms[-1] >= ms[-2]
        assert np.all(np.diff(L, axis=1) > 0)


def test_lloyd_step_levels_are_weighted_centroids_and_midpoints():
    rng = np.random.default_rng(4)
    x, w = _data(rng, R=2, K=256)
    T0 = np.tile(lloyd.init_thresholds(2), (2, 1))
    L0 = np.tile(lloyd.init_levels(2), (2, 1))
    L, T1, mse = lloyd.lloyd_step(x, w, T0, L0)
    for i in range(2):
        for k in range(4):
            lo = -np.inf if k == 0 else T0[i, k - 1]
            hi = np.inf if k == 3 else T0[i, k]
            sel = (x[i] > lo) & (x[i] <= hi)
            num = math.fsum(w[i, sel] * x[i, sel])
            den = math.fsum(w[i, sel])
            assert abs(L[i, k] - num / den) < 1e-12
        assert np.allclose(T1[i], (L[i, :-1] + L[i, 1:]) / 2, rtol=0, atol=0)


def test_lloyd_two_clusters_closed_form():
    # 1 bit, data at two points with weights: the centroids are the points
    x = np.array([[-0.5] * 64 + [0.25] * 64])
    w = np.ones_like(x)
    L, T, it = lloyd.learn(x, w, 1)
    assert np.allclose(L, [[-0.5, 0.25]]) and np.allclose(T, [[-0.125]])


def test_nf_init_tables():
    # the initial tables follow the NF construction at 2, 3 and 4 bits
    assert np.array_equal(lloyd.init_levels(4).astype(np.float32), nf4.levels())
    for b in (2, 3):
        L = lloyd.init_levels(b)
        assert L.size == 1 << b and L[0] == -1 and L[-1] == 1 and 0.0 in L
        assert np.all(np.diff(L) > 0)
    assert np.array_equal(lloyd.init_thresholds(1), [0.0])


def test_learn_codebooks_outputs_valid_tables():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    bits = np.array([1, 2, 3, 4, 1, 2, 3, 4])
    L, T = lloyd.learn_codebooks(W, bits)
    for i, b in enumerate(bits):
        n = 1 << b
        assert np.all(np.diff(L[i, :n]) > 0)
        assert np.all(np.diff(T[i, :n - 1]) > 0)
        assert np.all(T[i, :n - 1] >= L[i, :n - 1]) and np.all(T[i, :n - 1] < L[i, 1:n])


# ---- the weighted error and the stop rule, pinned by hand-derived values ----
# LowRA page, section 5: each channel minimises its own mean squared error,
# weighted by the absmax of the block an element lies in; an iteration takes
# the weighted centroid of every bin, then midpoints; the learner stops when
# the error stops decreasing and returns the last pair computed. The values
# below are exact dyadic fractions derived by hand (and checked in exact
# rational arithmetic), not outputs of the oracle.

def test_lloyd_step_error_hand_computed():
    # 1 bit from threshold 0 and levels {-1, +1}; two elements carry weight 1
    # (a block of absmax 1), two weight 2, one weight 4.
    x = np.array([[-0.75, -0.25, 0.25, 0.5, 1.0]])
    w = np.array([[1.0, 1.0, 2.0, 2.0, 4.0]])
    L, T1, mse = lloyd.lloyd_step(x, w, np.array([[0.0]]), np.array([[-1.0, 1.0]]))
    # bins {-0.75, -0.25} and {0.25, 0.5, 1.0}:
    # L0 = (-0.75 - 0.25) / 2 = -0.5, L1 = (0.5 + 1 + 4) / 8 = 0.6875
    assert L.tolist() == [[-0.5, 0.6875]]
    assert T1.tolist() == [[0.09375]]
    # squared errors against the new levels, weighted:
    # 1/16 + 1/16 + 2 (7/16)^2 + 2 (3/16)^2 + 4 (5/16)^2 = 31/32, over sum w = 10
    # (unweighted, the same errors give 0.08984375; weighted against the
    # previous levels {-1, +1}, 0.225)
    assert mse.tolist() == [0.096875]


def test_lloyd_step_error_is_weighted_fsum_over_elements():
    rng = np.random.default_rng(11)
    K = 192
    x = np.clip(rng.standard_normal((3, K)) / 2.5, -1, 1)
    w = np.repeat(np.array([[0.25, 1.0, 3.5], [2.0, 0.5, 1.0], [1.0, 1.0, 8.0]]), 64, axis=1)
    for b in (1, 2, 3, 4):
        T0 = np.tile(lloyd.init_thresholds(b), (3, 1))
        L0 = np.tile(lloyd.init_levels(b), (3, 1))
        L, _, mse = lloyd.lloyd_step(x, w, T0, L0)
        for i in range(3):
            # element by element: its bin by scanning the thresholds from the
            # bottom, its error against that bin's new level
            terms, wsum = [], []
            for k in range(K):
                j = 0
                while j < T0.shape[1] and x[i, k] > T0[i, j]:
                    j += 1
                terms.append(w[i, k] * (x[i, k] - L[i, j]) ** 2)
                wsum.append(w[i, k])
            want = math.fsum(terms) / math.fsum(wsum)
            assert abs(mse[i] - want) <= 1e-12 * want


def test_lloyd_stop_iteration_on_a_discriminating_row():
    # Eight values in sixteenths with block weights 1, 2, 1, 8, 2, 2, 1, 8.
    # In exact arithmetic the weighted learner moves through
    #   it 1: L = (-77/192, 15/26),  error 83807/998400
    #   it 2: L = (-75/224, 59/88),  error 14519/197120
    #   it 3: L = (-71/256, 19/24),  error 6079/102400
    #   it 4: the same bins again, the same error -> stop after 4 iterations.
    # Other readings stop elsewhere on this row: unweighted centroids and error
    # after 2, the unweighted error at the previous levels after 3, the
    # weighted error at the previous levels after 5.
    x = np.array([[-15, -12, -6, -4, 1, 2, 10, 13]]) / 16.0
    w = np.array([[1.0, 2.0, 1.0, 8.0, 2.0, 2.0, 1.0, 8.0]])
    hist = []
    L, T, it = lloyd.learn(x, w, 1, history=hist)
    assert it.tolist() == [4]
    want = [83807 / 998400, 14519 / 197120, 6079 / 102400, 6079 / 102400]
    got = [float(m[0]) for _, m in hist]
    assert len(got) == 4
    for g, v in zip(got, want):
        assert abs(g - v) <= 1e-15 * v
    assert abs(L[0, 0] - (-71 / 256)) < 1e-16 and abs(L[0, 1] - 19 / 24) < 1e-15
    assert abs(T[0, 0] - (-71 / 256 + 19 / 24) / 2) < 1e-15
    # stopping one iteration later or earlier would return other levels
    L3, _, it3 = lloyd.learn(x, w, 1, max_iters=2)
    assert it3.tolist() == [2] and abs(L3[0, 1] - 59 / 88) < 1e-15


def test_lloyd_empty_bin_keeps_previous_level():
    # 2 bits from NF2: levels (-1, 0, l2, 1), thresholds their midpoints
    # (-0.5, l2/2, (l2+1)/2) with l2 ~ 0.436. The data fill bins 1 and 3 only;
    # bins 0 and 2 are empty and keep their starting levels exactly.
    L0 = lloyd.init_levels(2)
    x = np.array([[0.125, 0.1875, 0.875, 1.0]])
    w = np.array([[1.0, 3.0, 2.0, 2.0]])
    hist = []
    L, T, it = lloyd.learn(x, w, 2, history=hist)
    l1 = (0.125 + 3 * 0.1875) / 4          # 0.171875
    l3 = (2 * 0.875 + 2 * 1.0) / 4         # 0.9375
    assert L[0, 0] == L0[0] == -1.0 and L[0, 2] == L0[2]
    assert L[0, 1] == l1 and L[0, 3] == l3
    assert np.array_equal(T[0], (L[0, :-1] + L[0, 1:]) / 2)
    # the bins are the same in the second iteration, so it stops there
    assert it.tolist() == [2]
    err = (1 * (0.125 - l1) ** 2 + 3 * (0.1875 - l1) ** 2 + 2 * 0.0625 ** 2 + 2 * 0.0625 ** 2) / 8
    assert abs(float(hist[0][1][0]) - err) <= 1e-15 * err
