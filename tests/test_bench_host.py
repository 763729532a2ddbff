"""Host-side checks of bench.py: the algorithmic work it divides by, and its
one-GPU guard (runs without a GPU).

The byte counts follow from the storage format alone: a weight is read as
float32 (4 B) and written as packed NF4 (1/2 B), one float32 absmax per
64-block (QLoRA page, NF4 section), and with double quantization one 8-bit
code per block, one float32 scale per 256 blocks and one float32 mean
(QLoRA page, double-quantization section); the dequantized weight is bf16.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class Layer:
    def __init__(self, N, K, r, M):
        self.N, self.K, self.r, self.M = N, K, r, M


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (28672, 8192)])
def test_codec_bytes_follow_the_format(bench, N, K):
    n = N * K
    b = bench.codec_bytes(Layer(N, K, 16, 1), 1)
    # quantize: 4 B read + 1/2 B written per weight, 4 B per 64 weights
    assert b["quantize"] * 64 == n * (4 * 64 + 32 + 4)
    # profiling pass: the float32 weight once
    assert b["profile"] == 4 * n
    consts = n // 64 + 4 * ((n // 64 + 255) // 256) + 4
    assert b["dequant"] == n // 2 + consts + 2 * n
    assert b["double_quant"] == 4 * (n // 64) + consts
    # the two in one call: the float32 constants and the codes in, the
    # double-quantized constants and the bf16 weight out
    assert b["double_quant_dequant"] == 4 * (n // 64) + n // 2 + consts + 2 * n
    # decode GEMV at M tokens (t given): packed weight + X + B + H + t
    for M in (1, 4, 16):
        g = bench.codec_bytes(Layer(N, K, 16, M), M)["gemv"]
        assert g == n // 2 + consts + 2 * K * M + 2 * N * 16 + 2 * N * M + 4 * M * 16


def test_q_proj_decode_figures(bench):
    # the 4096^2 and 28672 x 8192 layers in whole bytes
    q = bench.codec_bytes(Layer(4096, 4096, 16, 2048))
    assert q["quantize"] == 76_546_048 and q["dequant"] == 42_209_284
    d = bench.codec_bytes(Layer(28672, 8192, 16, 1), 1)
    assert d["gemv"] - (2 * 8192 + 2 * 28672 * 16 + 2 * 28672 + 4 * 16) == 121_167_876


def test_layer_flops(bench):
    M, N, K, r = 2048, 4096, 4096, 16
    f = bench.layer_flops(Layer(N, K, r, M), M)
    assert f["fwd_gemm"] == 2 * M * N * K + 2 * M * N * r     # X W'^T + (s t) B^T in one GEMM
    assert f["lora_down"] == 2 * M * K * r                     # t = X A^T
    # backward: grad_X = G W' + s u A, u = G B, dB = s G^T t, dA = s u^T X
    assert f["bwd"] == 2 * M * N * K + 2 * M * K * r + 2 * M * N * r + 2 * M * N * r + 2 * M * K * r


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("steps", [1, 4, 5, 9, 20, 21, 200, 1000])
def test_kernel_event_stride_times_enough_launches(bench, steps):
    s = bench.kernel_event_stride(steps)
    timed = len(range(0, steps, s))
    assert 1 <= s <= 4
    # at least 5 launches are timed whenever the window has 5 steps
    assert timed >= min(5, steps)


@pytest.mark.parametrize("N,K", [(1024, 1024), (4096, 4096), (11008, 4096), (28672, 8192)])
def test_codec_rotation_defeats_the_infinity_cache(bench, N, K):
    # every rotated codec arm moves at least 1 GiB per pass over its copies
    # (four times the 256 MB cache), the dequant arm (2.5 B per weight) being
    # the smallest
    k = bench.rotation_count(N * K)
    b = bench.codec_bytes(Layer(N, K, 16, 1))
    for arm in ("quantize", "profile", "dequant"):
        assert k * b[arm] >= 1 << 30
    assert (k - 1) * (5 * N * K // 2) < 1 << 30   # and no more copies than that needs


def test_lowra_decode_bytes(bench):
    """Codebook decode GEMV: the bit-planes (K b / 8 bytes per row), one E4M3
    code per 64-block, one float32 scale per 256 blocks and the mean, the
    widths (1 B per row), offsets (8 B per row + 1) and levels (16 float32 per
    row), then X, t, B in and H out (LowRA page, section 4.1: per-channel
    widths and mappings)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import synthetic as syn
    L = syn.LAYERS["lowra"]
    lb = bench.lowra_bytes(syn, L)
    n_b = L.N * L.K // 64
    planes = L.K * (256 * 4 + 512 * 3 + 1280 * 2 + 2048 * 1) // 8     # 1.75 bits per weight
    assert planes == L.N * L.K * 7 // 32
    w = planes + n_b + 4 * (n_b // 256) + 4 + L.N + 8 * (L.N + 1) + 64 * L.N
    assert lb["weight"] == w
    assert lb["gemv"](16) == w + 2 * L.K * 16 + 4 * 16 * L.r + 2 * L.N * L.r + 2 * L.N * 16
