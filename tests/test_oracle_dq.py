"""Pins of the oracle's 8-bit float, double quantization and size closed
forms (QLoRA page, Contribution 2) against the OCP E4M3 definition, exact
arithmetic and the page's printed numbers."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8, dq, sizes


def _all_e4m3_values():
    # From the OCP 8-bit float specification: E4M3, bias 7, subnormal step
    # 2^-9, largest finite 448 (S.1111.110), S.1111.111 is NaN.
    vals = {}
    for code in range(128):
        e, m = code >> 3, code & 7
        if e == 15 and m == 7:
            continue
        v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        vals[code] = v
    return vals


def test_e4m3_decode_spec_points():
    d = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x38] == 1.0 and d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    for code, v in _all_e4m3_values().items():
        assert Fraction(float(d[code])) == v


def _bruteforce_encode(x):
    vals = _all_e4m3_values()
    xf = Fraction(float(x))
    a = abs(xf)
    best = min(vals.items(), key=lambda kv: (abs(kv[1] - a), kv[0] & 1))
    return best[0] | (0x80 if np.signbit(np.float32(x)) else 0)


def test_e4m3_encode_against_nearest_even_bruteforce():
    vals = sorted(_all_e4m3_values().values())
    pts = []
    for i, v in enumerate(vals):
        pts.append(float(v))
        if i + 1 < len(vals):
            mid = np.float32(float((v + vals[i + 1]) / 2))   # midpoints are float32-exact here
            pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    rng = np.random.default_rng(1)
    pts += list(rng.uniform(-448, 448, 2000)) + list(rng.uniform(-0.03, 0.03, 2000))
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts, np.array([0.0, -0.0], dtype=np.float32)])
    pts = pts[np.abs(pts) <= 448]
    got = fp8.e4m3_encode(pts)
    for x, g in zip(pts, got):
        assert g == _bruteforce_encode(x), (x, g)


def test_size_closed_forms_match_page():
    # 8/64 + 32/(64*256) ~= 0.127 bit/param, saving 0.373 vs 32/64 = 0.5
    b = sizes.constant_bits_per_param()
    assert b == Fraction(8, 64) + Fraction(32, 16384)
    assert round(float(b), 3) == 0.127
    assert sizes.constant_bits_per_param(double_quant=False) == Fraction(1, 2)
    assert round(0.5 - float(b), 3) == 0.373
    # 30B parameters: 30e9 * 0.373 / 8 ~= 1.40 GB
    assert round(sizes.saving_bytes(30e9) / 1e9, 2) == 1.40
    # byte counts of one layer: 4-bit codes + 1 B code + 4 B per 256 + 4 B mean
    s = sizes.storage(28672, 8192)
    assert s["code_bytes"] == 117440512 and s["const_bytes"] == 3670016 + 57344 + 4


def test_tree_mean_within_one_ulp_of_exact():
    rng = np.random.default_rng(2)
    for n in (1, 7, 256, 257, 1000, 4099):
        c = np.abs(rng.standard_normal(n) * 0.05).astype(np.float32) + np.float32(0.01)
        mu = dq.tree_mean(c)
        exact = Fraction(math.fsum(float(x) for x in c)) / n
        ulp = Fraction(float(np.spacing(np.float32(mu))))
        assert abs(Fraction(float(mu)) - exact) <= ulp


def test_tree_mean_order_is_pairwise_tree():
    # [2^53, 1, 1, -2^53]: the balanced tree adds (2^53 + 1) -> 2^53 (tie to
    # even) and (1 - 2^53) exactly, then gives 1. Left to right gives 0 and
    # ((a + (b + c)) + d) gives 2, so only the pairwise tree returns 1.
    big = float(2 ** 53)
    v = np.array([big, 1.0, 1.0, -big])
    assert dq.pairwise_sum_f64(v) == 1.0


def test_double_quant_invariants_and_bound():
    rng = np.random.default_rng(4)
    c = np.abs(rng.standard_normal(3000) * 0.02 + 0.03).astype(np.float32) + np.float32(1e-3)
    code8, s2, mu = dq.double_quant(c)
    assert code8.size == 3000 and s2.size == 12
    cp = dq.dq_decode(code8, s2, mu)
    d = (c - mu).astype(np.float32)
    for J in range(12):
        blk = code8[256 * J:256 * (J + 1)]
        # every block with a2 > 0 uses a +-448 code
        assert np.any((blk == 0x7E) | (blk == 0xFE))
    s2b = np.repeat(s2, 256)[:3000].astype(np.float64)
    bound = np.maximum(np.abs(d) * 2.0 ** -4, 2.0 ** -10 * s2b) + 2 * np.spacing(np.abs(c))
    assert np.all(np.abs(c.astype(np.float64) - cp) <= bound)


def test_double_quant_constant_block_decodes_to_mean():
    c = np.full(300, 0.0125, dtype=np.float32)
    code8, s2, mu = dq.double_quant(c)
    assert mu == np.float32(0.0125)
    assert np.all(code8 == 0) and np.all(s2 == 0)
    assert np.all(dq.dq_decode(code8, s2, mu) == np.float32(0.0125))


def test_golden_printed_numbers():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "qlora_printed_numbers.json")))
    blk, dqb = g["fp32_constant_per_weights"], g["dq_blocksize"]
    assert float(sizes.constant_bits_per_param(blk, dqb, False)) == g["first_level_bits_per_param"]
    assert round(float(sizes.constant_bits_per_param(blk, dqb, True)), 3) == g["dq_bits_per_param_3dp"]
    assert round(0.5 - float(sizes.constant_bits_per_param(blk, dqb, True)), 3) == g["dq_saving_bits_per_param_3dp"]
    assert round(sizes.saving_bytes(g["model_params_for_saving"], blk, dqb) / 1e9, 2) == g["saving_GB_2dp"]
    from oracle import nf4
    assert nf4.levels().size == g["nf4_levels_total"] == g["nf4_negative_quantiles"] + g["nf4_positive_quantiles"] - 1
