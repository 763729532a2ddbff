"""Property tests of the codec kernels and geometry reruns on the GPU.

Property tests: seeded random shapes (N rows, K a multiple of 64) filled
block by block with random edge content -- all-zero and signed-zero blocks,
constant blocks, subnormal blocks, a single outlier, +-absmax ties, values
exactly on the NF4 midpoints times the block constant and their float32
neighbours -- quantized, double quantized and dequantized on the GPU and
compared bit for bit with the oracle (QLoRA page, Contributions 1 and 2:
absmax per 64-block, nearest NF4 value, 8-bit constants over 256-blocks).
The same for the per-channel codebook quantizer with random widths and
thresholds (LowRA page, sections 3 and 4.1).

Geometry reruns: the same data processed by launches of a different shape
(row ranges of the weight in separate calls, so grids and workgroup-to-block
maps change) must give byte-identical results; double quantization (whose
mean needs all constants) must repeat exactly run to run and from another
address.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import nf4, dq, codebook

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


def random_edge_weight(rng, N, K):
    """N x K float32 with a random kind of content per 64-block."""
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    flat = W.reshape(-1, 64)
    t = nf4.thresholds()
    for b in range(flat.shape[0]):
        kind = rng.integers(0, 9)
        if kind == 0:
            flat[b] = 0.0
        elif kind == 1:
            flat[b] = np.where(rng.random(64) < 0.5, np.float32(-0.0), np.float32(0.0))
        elif kind == 2:
            flat[b] = np.float32(rng.uniform(-0.1, 0.1))
        elif kind == 3:
            flat[b] = (rng.standard_normal(64) * 1e-39).astype(np.float32)     # subnormal
        elif kind == 4:
            flat[b, rng.integers(0, 64)] = np.float32(rng.uniform(1, 100)) * rng.choice([-1, 1])
        elif kind == 5:
            c = np.float32(rng.uniform(0.001, 0.5))
            flat[b, rng.integers(0, 64)] = c
            flat[b, rng.integers(0, 64)] = -c                                  # +-absmax tie
        elif kind == 6:
            c = np.float32(rng.uniform(0.001, 0.5))
            ti = t[rng.integers(0, 15, 40)]
            v = (ti * c).astype(np.float32)
            v = np.where(rng.random(40) < 0.33, np.nextafter(v, np.float32(2)),
                         np.where(rng.random(40) < 0.5, np.nextafter(v, np.float32(-2)), v))
            flat[b, :40] = v
            flat[b, 40:63] = (c * rng.uniform(-1, 1, 23)).astype(np.float32)
            flat[b, 63] = c
        # kinds 7, 8: plain Gaussian block
    return W


CASES = [(int(n), int(64 * k)) for n, k in zip(np.random.default_rng(2024).integers(1, 300, 12),
                                                np.random.default_rng(2025).integers(1, 40, 12))]


@pytest.mark.parametrize("N,K", CASES)
def test_random_shapes_quantize_dq_dequant_bit_exact(lq, torch, N, K):
    rng = np.random.default_rng(N * 1000 + K)
    W = random_edge_weight(rng, N, K)
    codes, absmax = lq.quantize_nf4(dev(torch, W))
    packed, c = nf4.quantize(W)
    assert np.array_equal(host(absmax), c)
    assert np.array_equal(host(codes), packed)
    q, s2, mu = lq.double_quant(absmax)
    oq, os2, omu = dq.double_quant(c)
    assert host(mu)[0] == omu and np.array_equal(host(s2), os2) and np.array_equal(host(q), oq)
    for double in (False, True):
        qw = lq.QWeight(N, K, codes, absmax=None if double else absmax, absmax_q=q if double else None,
                        dq_scale=s2 if double else None, dq_mean=mu if double else None)
        got = host(lq.dequant(qw).contiguous().view(torch.int16)).view(np.uint16)
        cp = dq.dq_decode(oq, os2, omu) if double else c
        assert np.array_equal(got, nf4.dequant(packed, cp, W.shape, as_bits=True))


@pytest.mark.parametrize("seed", range(6))
def test_random_codebook_quantize_bit_exact(lq, torch, seed):
    rng = np.random.default_rng(700 + seed)
    N, K = int(rng.integers(1, 200)), int(64 * rng.integers(1, 24))
    W = random_edge_weight(rng, N, K)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    T = np.full((N, 15), 3.0, dtype=np.float32)
    for i, b in enumerate(bits):
        T[i, :(1 << b) - 1] = np.sort(rng.uniform(-1, 1, (1 << b) - 1)).astype(np.float32)
    codes, absmax, row_off = lq.quantize_codebook(dev(torch, W), dev(torch, bits), dev(torch, T))
    packed, c, _ = codebook.quantize(W, bits, T)
    assert np.array_equal(host(absmax), c)
    assert np.array_equal(host(codes)[:packed.size], packed)


# ---- geometry reruns ------------------------------------------------------

def test_quantize_row_ranges_match_whole(lq, torch):
    rng = np.random.default_rng(31)
    N, K = 777, 448
    W = dev(torch, random_edge_weight(rng, N, K))
    codes, absmax = lq.quantize_nf4(W)
    for n1 in (1, 100, 383, 776):
        ca, aa = lq.quantize_nf4(W[:n1])
        cb, ab = lq.quantize_nf4(W[n1:])
        assert torch.equal(torch.cat([ca, cb]), codes) and torch.equal(torch.cat([aa, ab]), absmax)


@pytest.mark.parametrize("double", [False, True])
def test_dequant_row_ranges_match_whole(lq, torch, double):
    rng = np.random.default_rng(32)
    N, K = 1024, 256          # 4 blocks per row: 64 rows per 256-constant group
    W = dev(torch, random_edge_weight(rng, N, K))
    qw = lq.QWeight.from_weight(W, double_quantize=double)
    whole = lq.dequant(qw)
    for n1 in (64, 512, 960):
        parts = []
        for r0, r1 in ((0, n1), (n1, N)):
            b0, b1 = r0 * K // 64, r1 * K // 64
            sub = lq.QWeight(r1 - r0, K, qw.codes[r0 * K // 2:r1 * K // 2],
                             absmax=None if double else qw.absmax[b0:b1],
                             absmax_q=qw.absmax_q[b0:b1] if double else None,
                             dq_scale=qw.dq_scale[b0 // 256:(b1 + 255) // 256] if double else None,
                             dq_mean=qw.dq_mean if double else None)
            parts.append(lq.dequant(sub))
        assert torch.equal(torch.cat(parts).view(torch.int16), whole.view(torch.int16))


def test_double_quant_repeats_exactly(lq, torch):
    rng = np.random.default_rng(33)
    c = dev(torch, np.abs(rng.standard_normal(300000) * 0.02 + 0.05).astype(np.float32))
    first = lq.double_quant(c)
    other = torch.empty(c.numel() + 64, dtype=torch.float32, device="cuda")[64:]
    other.copy_(c)                      # same values at another address
    for src in (c, c, other):
        again = lq.double_quant(src)
        assert all(torch.equal(a, b) for a, b in zip(first, again))


def test_codebook_row_ranges_match_whole(lq, torch):
    rng = np.random.default_rng(34)
    N, K = 301, 320
    W = dev(torch, random_edge_weight(rng, N, K))
    bits = rng.integers(1, 5, N).astype(np.uint8)
    T = np.full((N, 15), 3.0, dtype=np.float32)
    for i, b in enumerate(bits):
        T[i, :(1 << b) - 1] = np.sort(rng.uniform(-1, 1, (1 << b) - 1)).astype(np.float32)
    bd, Td = dev(torch, bits), dev(torch, T)
    codes, absmax, row_off = lq.quantize_codebook(W, bd, Td)
    off = host(row_off)
    for n1 in (1, 150, 300):
        ca, aa, _ = lq.quantize_codebook(W[:n1], bd[:n1], Td[:n1])
        cb, ab, _ = lq.quantize_codebook(W[n1:], bd[n1:], Td[n1:])
        assert torch.equal(ca[:off[n1]], codes[:off[n1]]) and torch.equal(cb[:off[N] - off[n1]], codes[off[n1]:off[N]])
        assert torch.equal(torch.cat([aa, ab]), absmax)


def test_forward_row_ranges_match_whole(lq, torch):
    """The dequant-GEMM computes each output from its own row of X in a fixed
    k order, whatever tile the row falls in: splitting the tokens over two
    calls (other grids and tile positions) gives the same bits."""
    L = syn.small_layer(384, 512, 600, 16, 32.0, 35)
    W, X, A, B = syn.weight(L), syn.activations(L), syn.lora_a(L), syn.lora_b(L)
    qw = lq.QWeight.from_weight(dev(torch, W))
    bf = lambda bits: dev(torch, bits.view(np.int16)).view(torch.bfloat16)
    Xd, Ad, Bd = bf(X.bits), bf(A.bits), bf(B.bits)
    H, t = lq.qlora_forward(qw, Xd, Ad, Bd, 32.0, out_dtype=torch.float32)
    for m1 in (17, 256, 300, 583):
        Ha, ta = lq.qlora_forward(qw, Xd[:m1].contiguous(), Ad, Bd, 32.0, out_dtype=torch.float32)
        Hb, tb = lq.qlora_forward(qw, Xd[m1:].contiguous(), Ad, Bd, 32.0, out_dtype=torch.float32)
        assert torch.equal(torch.cat([Ha, Hb]), H) and torch.equal(torch.cat([ta, tb]), t)


@pytest.mark.parametrize("spacing", ["wide", "close"])
def test_codebook_quantize_at_thresholds(lq, torch, spacing):
    """Weights whose quotient w / c lands on one of the row's thresholds, or
    a few float32 steps either side of it (block constant c: the block's own
    absmax, stored in the block). Wide spacing (thresholds more than 1/64
    apart) takes the code search through the row's bin table and its exact
    fallback near a threshold; close spacing (two thresholds within 1/128)
    counts thresholds directly. Both must match the oracle bit for bit
    (LowRA page, section 4.1: thresholds per output channel)."""
    rng = np.random.default_rng(41 if spacing == "wide" else 42)
    N, K = 96, 512
    bits = np.tile(np.array([1, 2, 3, 4], dtype=np.uint8), N // 4)
    T = np.full((N, 15), 3.0, dtype=np.float32)
    W = np.zeros((N, K), dtype=np.float32)
    for i, b in enumerate(bits):
        nt = (1 << int(b)) - 1
        if spacing == "wide":
            t = np.sort(rng.uniform(-0.9, 0.9, nt))
            while nt > 1 and np.min(np.diff(t)) < 0.05:
                t = np.sort(rng.uniform(-0.9, 0.9, nt))
        else:
            t = np.sort(rng.uniform(-0.9, 0.9, nt))
            if nt > 1:
                t[1] = t[0] + 1.0 / 256          # two thresholds in one bin
                t = np.sort(t)
        T[i, :nt] = t.astype(np.float32)
        for blk in range(K // 64):
            c = np.float32(rng.uniform(0.01, 0.3))
            vals = []
            for tk in T[i, :nt]:
                w0 = np.float32(tk * c)
                vals += [w0, np.nextafter(w0, np.float32(1)), np.nextafter(w0, np.float32(-1)),
                         np.nextafter(np.nextafter(w0, np.float32(1)), np.float32(1))]
            vals = np.array(vals[:63], dtype=np.float32)
            W[i, blk * 64:blk * 64 + vals.size] = vals
            W[i, blk * 64 + vals.size:blk * 64 + 63] = (c * rng.uniform(-1, 1, 63 - vals.size)).astype(np.float32)
            W[i, blk * 64 + 63] = c
    codes, absmax, _ = lq.quantize_codebook(dev(torch, W), dev(torch, bits), dev(torch, T))
    packed, cc, _ = codebook.quantize(W, bits, T)
    assert np.array_equal(host(absmax), cc)
    assert np.array_equal(host(codes)[:packed.size], packed)
