"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact for codes, packed bytes, block constants, E4M3 codes and the
bfloat16 dequantized weight; relative Frobenius error <= 2e-3 for bfloat16
outputs of the GEMMs (H, grad_X) and <= 1e-4 for float32 outputs (H in
float32, t, dA, dB) against the float64 oracle.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import nf4, dq, layer, codebook, lloyd

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
F32_TOL = 1e-4


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


def bf16_dev(torch, bits):
    return dev(torch, bits.view(np.int16)).view(torch.bfloat16)


def bf16_to_f32(t):
    import torch
    bits = host(t.contiguous().view(torch.int16)).view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def oracle_qweight(W, double_quant=True):
    packed, c = nf4.quantize(W)
    if double_quant:
        code8, s2, mu = dq.double_quant(c)
        cp = dq.dq_decode(code8, s2, mu)
        return packed, c, (code8, s2, mu), cp
    return packed, c, None, c


# ---------------------------------------------------------------------------
# quantize
# ---------------------------------------------------------------------------
def edge_weight(rng, N, K):
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    flat = W.reshape(-1, 64)
    nb = flat.shape[0]
    flat[0] = 0.0                                   # all-zero block
    flat[1, ::2] = -0.0                             # signed zeros
    flat[2] = np.float32(3e-39) * rng.standard_normal(64).astype(np.float32)  # subnormal block
    flat[3] = np.float32(0.0123)                    # constant block
    flat[4, 7] = 5.0                                # one huge outlier
    t = nf4.thresholds()
    # exact midpoints and their neighbours for several block constants
    for b in range(5, min(nb, 40)):
        c = np.float32(rng.uniform(0.001, 0.2))
        vals = []
        for ti in t:
            w0 = np.float32(ti * c)
            vals += [w0, np.nextafter(w0, np.float32(1)), np.nextafter(w0, np.float32(-1))]
        vals = np.array(vals, dtype=np.float32)           # 45 values
        flat[b, :vals.size] = vals
        flat[b, vals.size:63] = (c * rng.uniform(-1, 1, 63 - vals.size)).astype(np.float32)
        flat[b, 63] = c
    return W


@pytest.mark.parametrize("shape", [(64, 64), (192, 320), (1000, 128), (37, 1024)])
def test_quantize_nf4_bit_exact(lq, torch, shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    W = edge_weight(rng, *shape) if shape[0] * shape[1] >= 64 * 64 else \
        (rng.standard_normal(shape) * 0.02).astype(np.float32)
    codes, absmax = lq.quantize_nf4(dev(torch, W))
    packed, c = nf4.quantize(W)
    assert np.array_equal(host(absmax), c)
    assert np.array_equal(host(codes), packed)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quantize_nf4_half_inputs(lq, torch, dtype):
    rng = np.random.default_rng(5)
    W32 = (rng.standard_normal((96, 256)) * 0.02).astype(np.float32)
    if dtype == "bf16":
        Wt = dev(torch, W32).to(torch.bfloat16)
    else:
        Wt = dev(torch, W32).to(torch.float16)
    Wexact = host(Wt.float())
    codes, absmax = lq.quantize_nf4(Wt)
    packed, c = nf4.quantize(Wexact)
    assert np.array_equal(host(absmax), c) and np.array_equal(host(codes), packed)


def test_quantize_threshold_windows(lq, torch):
    """Every float32 within +-2^15 ulps of each threshold (and of each level),
    in blocks that also hold 1.0 so the block constant is 1 and x = w."""
    t = nf4.thresholds()
    pts = []
    for v in list(t) + list(nf4.levels()[1:-1]):
        b = np.float32(v).view(np.int32)
        if v > 0:
            pts.append((b + np.arange(-32768, 32768, dtype=np.int32)).view(np.float32))
        else:
            mag = np.float32(-v).view(np.int32) if v < 0 else np.int32(0)
            m = mag + np.arange(-32768, 32768, dtype=np.int32)
            m = m[m >= 0]
            pts.append(-(m.view(np.float32)))
    x = np.concatenate(pts).astype(np.float32)
    x = x[np.abs(x) <= 1.0]
    n63 = (x.size + 62) // 63
    blocks = np.zeros((n63, 64), dtype=np.float32)
    flat = np.zeros(n63 * 63, dtype=np.float32)
    flat[:x.size] = x
    blocks[:, :63] = flat.reshape(n63, 63)
    blocks[:, 63] = 1.0
    blocks[1::2, 63] = -1.0
    W = blocks.reshape(n63, 64)
    codes, absmax = lq.quantize_nf4(dev(torch, W))
    packed, c = nf4.quantize(W)
    assert np.array_equal(host(absmax), c)
    assert np.array_equal(host(codes), packed)


@pytest.mark.parametrize("scaled", [False, True])
def test_quantize_strided_sweep(lq, torch, scaled):
    """Every 61st float32 bit pattern of [-1, 1] (about 35 M values: every
    exponent, mantissas at a prime stride), 63 per block with the block's
    absmax in the last slot. Unscaled: absmax 1, so x = w exactly. Scaled:
    each block multiplied by its own constant in [0.01, 0.05] (rounded to
    float32), so the kernel's reciprocal shortcut and its exact-quotient
    fallback both decide codes; the oracle divides."""
    one = np.float32(1.0).view(np.int32)
    pos = np.arange(0, one + 1, 61, dtype=np.int32).view(np.float32)
    x = np.concatenate([pos, -pos[1:]])
    n63 = (x.size + 62) // 63
    flat = np.zeros(n63 * 63, dtype=np.float32)
    flat[:x.size] = x
    W = np.empty((n63, 64), dtype=np.float32)
    W[:, :63] = flat.reshape(n63, 63)
    W[:, 63] = 1.0
    if scaled:
        c = np.random.default_rng(11).uniform(0.01, 0.05, n63).astype(np.float32)
        W = (W.astype(np.float64) * c[:, None]).astype(np.float32)
    codes, absmax = lq.quantize_nf4(dev(torch, W))
    packed, cref = nf4.quantize(W)
    assert np.array_equal(host(absmax), cref)
    assert np.array_equal(host(codes), packed)


# ---------------------------------------------------------------------------
# double quantization
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_b", [1, 255, 256, 1000, 16384, 262144, 262145, 300000])
def test_double_quant_bit_exact(lq, torch, n_b):
    """Codes, scales and the mean bit for bit. Up to 1024 blocks of 256
    (n_b <= 262144) the encoder forms the mean from the block sums itself;
    past that a separate tree reduction does (262145: 1025 block sums)."""
    rng = np.random.default_rng(n_b)
    c = np.abs(rng.standard_normal(n_b) * 0.02 + 0.05).astype(np.float32)
    if n_b > 300:
        c[256:512] = np.float32(0.04)               # one constant block
    q, s2, mu = lq.double_quant(dev(torch, c))
    oq, os2, omu = dq.double_quant(c)
    assert host(mu)[0] == omu
    assert np.array_equal(host(s2), os2)
    assert np.array_equal(host(q), oq)


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("double", [False, True])
def test_dequant_bit_exact(lq, torch, double):
    rng = np.random.default_rng(11)
    W = edge_weight(rng, 256, 512)
    qw = lq.QWeight.from_weight(dev(torch, W), double_quantize=double)
    got = bf16_to_f32(lq.dequant(qw))
    packed, c, dqp, cp = oracle_qweight(W, double)
    want = nf4.dequant(packed, cp, W.shape)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("N,K", [(8, 64), (300, 128), (1024, 1024), (4096, 4096), (4100, 4096)])
def test_double_quant_dequant(lq, torch, N, K):
    """Double quantization and dequantization in one call: the bits of the
    two calls in turn (one kernel after the block sums up to 1024 DQ blocks,
    4096 x 4096 being exactly that many; 4100 x 4096 has 1025 and runs the two
    calls' kernels), and up to 1 M weights the oracle's bits (edge blocks,
    a ragged last DQ block at 300 x 128)."""
    rng = np.random.default_rng(N + K)
    small = N * K <= 1 << 20
    W = edge_weight(rng, N, K) if small else (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, absmax = lq.quantize_nf4(dev(torch, W))
    q, s2, mu, Wd = lq.double_quant_dequant(codes, absmax, (N, K))
    q2, s22, mu2 = lq.double_quant(absmax)
    Wd2 = lq.dequant(lq.QWeight(N, K, codes, absmax_q=q2, dq_scale=s22, dq_mean=mu2))
    assert torch.equal(q, q2)
    assert torch.equal(s2.view(torch.int32), s22.view(torch.int32))
    assert torch.equal(mu.view(torch.int32), mu2.view(torch.int32))
    assert torch.equal(Wd.view(torch.int16), Wd2.view(torch.int16))
    if small:
        packed, c, (oq, os2, omu), cp = oracle_qweight(W, True)
        assert np.array_equal(host(q), oq)
        assert np.array_equal(host(s2), os2)
        assert host(mu)[0] == omu
        want = nf4.dequant(packed, cp, W.shape)
        assert np.array_equal(bf16_to_f32(Wd).view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# forward / backward
# ---------------------------------------------------------------------------
def make_layer(rng_seed, N, K, M, r, alpha):
    L = syn.small_layer(N, K, M, r, alpha, rng_seed)
    W = syn.weight(L)
    X = syn.activations(L)
    A = syn.lora_a(L)
    B = syn.lora_b(L)
    return L, W, X, A, B


def oracle_wd(W, double=True):
    packed, c, dqp, cp = oracle_qweight(W, double)
    return nf4.dequant(packed, cp, W.shape)


@pytest.mark.parametrize("N,K,M,r,alpha", [
    (384, 640, 300, 16, 32.0),     # ragged M, several tiles
    (1024, 1024, 16, 16, 32.0),    # the 1024x1024 workload (GEMV path)
    (520, 256, 17, 64, 16.0),      # just above the GEMV boundary, ragged N
    (256, 512, 1, 16, 32.0),       # single token
    (256, 512, 4, 24, 8.0),        # r not a multiple of 16
    (100, 256, 40, 16, 32.0),      # N % 8 != 0: element-wise epilogue
    (136, 192, 600, 40, 16.0),     # three M tiles, two LoRA steps (2r = 80)
    (256, 512, 16, 32, 8.0),       # GEMV forming t itself at its largest rank
    (300, 1088, 7, 17, 16.0),      # same, two column tiles of t, odd K/64, ragged N
    (200, 256, 9, 33, 16.0),       # rank just past that: t from the separate kernel
    (520, 4096, 40, 24, 16.0),     # GEMM path, t over four 64-column blocks per wave
    (8200, 4096, 5, 24, 16.0),     # t in four column parts, added (and stored) by the GEMV
    (8200, 2112, 3, 40, 16.0),     # t in two column parts (one ragged), three 16-wide tiles
])
def test_forward(lq, torch, N, K, M, r, alpha):
    L, W, X, A, B = make_layer(100 + M, N, K, M, r, alpha)
    qw = lq.QWeight.from_weight(dev(torch, W))
    Xd, Ad, Bd = bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits)
    H, t = lq.qlora_forward(qw, Xd, Ad, Bd, alpha)
    H32, _ = lq.qlora_forward(qw, Xd, Ad, Bd, alpha, out_dtype=torch.float32)
    Wd = oracle_wd(W)
    Href, tref = layer.forward(Wd, X.f32, A.f32, B.f32, alpha)
    assert layer.rel_frobenius(host(t), tref) <= 1e-5
    assert layer.rel_frobenius(bf16_to_f32(H), Href) <= BF16_TOL
    assert layer.rel_frobenius(host(H32), Href) <= F32_TOL


@pytest.mark.parametrize("M,K,r", [(1, 8, 16), (17, 24, 5), (33, 40, 128), (300, 72, 64), (64, 4096, 16),
                                   (16, 8256, 32)])
def test_lora_down_shapes(lq, torch, M, K, r):
    """t = X A^T for short and ragged contractions (K a multiple of 8 only,
    fewer columns than one 64-column block, K past a whole number of blocks)."""
    rng = np.random.default_rng(M * 7 + K + r)
    X = syn.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    A = syn.to_bf16_bits((rng.standard_normal((r, K)) * 0.02).astype(np.float32))
    t = lq.lora_down(bf16_dev(torch, X), bf16_dev(torch, A))
    B = np.zeros((8, r), np.float32)
    _, tref = layer.forward(np.zeros((8, K), np.float32), syn.bf16_bits_to_f32(X), syn.bf16_bits_to_f32(A), B,
                            float(r))
    assert layer.rel_frobenius(host(t), tref) <= 1e-5


@pytest.mark.parametrize("M,K,r", [(2050, 512, 16), (2048, 4096, 16), (4100, 256, 16), (1030, 1024, 64),
                                   (3000, 512, 128)])
def test_lora_down_many_rows(lq, torch, M, K, r):
    """t = X A^T with many 16-row groups and ragged M: every row is written
    once and matches the oracle, and repeated calls give the same bits."""
    rng = np.random.default_rng(M + 3 * K + r)
    X = syn.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    A = syn.to_bf16_bits((rng.standard_normal((r, K)) * 0.02).astype(np.float32))
    Xd, Ad = bf16_dev(torch, X), bf16_dev(torch, A)
    t1 = torch.full((M, r), float("nan"), dtype=torch.float32, device="cuda")
    t2 = torch.full((M, r), float("nan"), dtype=torch.float32, device="cuda")
    lq.lora_down(Xd, Ad, t1)
    lq.lora_down(Xd, Ad, t2)
    assert torch.equal(t1, t2)
    _, tref = layer.forward(np.zeros((8, K), np.float32), syn.bf16_bits_to_f32(X), syn.bf16_bits_to_f32(A),
                            np.zeros((8, r), np.float32), float(r))
    assert layer.rel_frobenius(host(t1), tref) <= 1e-5


def test_forward_gemm_and_gemv_agree_at_boundary(lq, torch, monkeypatch):
    L, W, X, A, B = make_layer(7, 512, 1024, 16, 16, 32.0)
    qw = lq.QWeight.from_weight(dev(torch, W))
    args = (qw, bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits), 32.0)
    H1, _ = lq.qlora_forward(*args, out_dtype=torch.float32)
    monkeypatch.setenv("LQ_FORCE_PATH", "gemm")
    H2, _ = lq.qlora_forward(*args, out_dtype=torch.float32)
    Href, _ = layer.forward(oracle_wd(W), X.f32, A.f32, B.f32, 32.0)
    assert layer.rel_frobenius(host(H1), Href) <= F32_TOL
    assert layer.rel_frobenius(host(H2), Href) <= F32_TOL


@pytest.mark.parametrize("r", [8, 12, 40, 64, 128])
def test_lora_segment_load_paths(lq, torch, r):
    """The LoRA segment of both dequant-GEMMs (QLoRA page, introduction: the
    s t B^T and s u A terms) reads t / u with 16-byte loads when r % 8 == 0 and
    the array is 16-byte aligned, element by element otherwise. The same values
    at a 4-byte offset (legal: t and u need only their natural alignment) take
    the element path: outputs bit-identical to the aligned call, and both
    against the oracle. r = 12 takes the element path either way."""
    N, K, M, alpha = 264, 320, 300, 16.0
    rng = np.random.default_rng(7100 + r)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = syn.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    G = syn.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    A = syn.to_bf16_bits((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    B = syn.to_bf16_bits((rng.standard_normal((N, r)) * 0.05).astype(np.float32))
    t = rng.standard_normal((M, r)).astype(np.float32)
    u = rng.standard_normal((M, r)).astype(np.float32)
    qw = lq.QWeight.from_weight(dev(torch, W))
    Xd, Gd, Ad, Bd = (bf16_dev(torch, a) for a in (X, G, A, B))

    def placed(a, off):
        buf = torch.zeros(a.size + 4, dtype=torch.float32, device="cuda")
        v = buf[off:off + a.size].view(a.shape)
        v.copy_(torch.from_numpy(a))
        return v

    t0, t1, u0, u1 = placed(t, 0), placed(t, 1), placed(u, 0), placed(u, 1)
    assert t0.data_ptr() % 16 == 0 and t1.data_ptr() % 16 == 4
    H0 = lq.dequant_gemm(qw, Xd, t0, Bd, alpha, out_dtype=torch.float32)
    H1 = lq.dequant_gemm(qw, Xd, t1, Bd, alpha, out_dtype=torch.float32)
    gx0 = lq.dequant_gemm_t(qw, Gd, u0, Ad, alpha)
    gx1 = lq.dequant_gemm_t(qw, Gd, u1, Ad, alpha)
    torch.cuda.synchronize()
    assert torch.equal(H0, H1) and torch.equal(gx0, gx1)
    Wd = oracle_wd(W).astype(np.float64)
    s = alpha / r
    Xf, Gf = syn.bf16_bits_to_f32(X).astype(np.float64), syn.bf16_bits_to_f32(G).astype(np.float64)
    Af, Bf = syn.bf16_bits_to_f32(A).astype(np.float64), syn.bf16_bits_to_f32(B).astype(np.float64)
    Href = Xf @ Wd.T + s * (t.astype(np.float64) @ Bf.T)
    gref = Gf @ Wd + s * (u.astype(np.float64) @ Af)
    assert layer.rel_frobenius(host(H0), Href) <= F32_TOL
    assert layer.rel_frobenius(bf16_to_f32(gx0), gref) <= BF16_TOL


@pytest.mark.parametrize("N,K,M,r,double", [
    (16384, 256, 16, 16, True),    # 4 row groups per workgroup, K/64 not a multiple of 16
    (24576, 1024, 2, 16, True),    # 4 row groups at M <= 4
    (8200, 2048, 16, 24, True),    # 2 row groups, the last workgroup half past N
    (12288, 640, 1, 16, False),    # 2 row groups, float32 constants, odd K/64
    (4100, 8192, 16, 64, True),    # 1 row group, 16 + 4 rows past a whole workgroup
    (64, 20480, 3, 16, True),      # K past two row groups' constant table
    (40, 17024, 5, 8, False),      # same, K/64 not a multiple of 16, ragged N
])
def test_decode_gemv_row_groups(lq, torch, monkeypatch, N, K, M, r, double):
    """The decode kernel at every row-group count it launches with, forming t
    itself (grids of at most 256 workgroups, r <= 32) or reading it, against
    the oracle and against the GEMM path on the same inputs."""
    rng = np.random.default_rng(N + K + M)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = syn.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    A = syn.to_bf16_bits((rng.standard_normal((r, K)) * 0.02).astype(np.float32))
    B = syn.to_bf16_bits((rng.standard_normal((N, r)) * 0.02).astype(np.float32))
    qw = lq.QWeight.from_weight(dev(torch, W), double_quantize=double)
    args = (qw, bf16_dev(torch, X), bf16_dev(torch, A), bf16_dev(torch, B), 32.0)
    H, t = lq.qlora_forward(*args)
    H32, _ = lq.qlora_forward(*args, out_dtype=torch.float32)
    Href, tref = layer.forward(oracle_wd(W, double), syn.bf16_bits_to_f32(X), syn.bf16_bits_to_f32(A),
                               syn.bf16_bits_to_f32(B), 32.0)
    assert layer.rel_frobenius(host(t), tref) <= 1e-5
    assert layer.rel_frobenius(bf16_to_f32(H), Href) <= BF16_TOL
    assert layer.rel_frobenius(host(H32), Href) <= F32_TOL
    monkeypatch.setenv("LQ_FORCE_PATH", "gemm")
    Hg, _ = lq.qlora_forward(*args, out_dtype=torch.float32)
    assert layer.rel_frobenius(host(Hg), Href) <= F32_TOL


@pytest.mark.parametrize("M", [5, 300])
def test_unit_vector_probe_bit_exact(lq, torch, M):
    """X rows = e_k, B = 0: H[m, :] = W'[:, k_m] exactly (float32 output)."""
    rng = np.random.default_rng(3)
    N, K = 384, 512
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ks = rng.integers(0, K, M)
    X = np.zeros((M, K), dtype=np.uint16)
    X[np.arange(M), ks] = 0x3F80       # 1.0 in bf16
    A = syn.to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32))
    B = np.zeros((N, 16), dtype=np.uint16)
    qw = lq.QWeight.from_weight(dev(torch, W))
    H, _ = lq.qlora_forward(qw, bf16_dev(torch, X), bf16_dev(torch, A), bf16_dev(torch, B), 32.0,
                            out_dtype=torch.float32)
    Wd = oracle_wd(W)
    assert np.array_equal(host(H), Wd[:, ks].T)


@pytest.mark.parametrize("N,K,M,r,alpha", [
    (384, 640, 300, 16, 32.0),
    (512, 256, 96, 64, 16.0),
    (264, 320, 33, 24, 8.0),       # N % 64 != 0, M % 32 != 0, hi/lo rows kept apart
    (192, 256, 50, 128, 16.0),     # largest rank: eight 16-wide tiles of t and u
    (136, 192, 77, 40, 16.0),      # 2r = 80: three 32-row product tiles
    (2056, 2048, 70, 16, 32.0),    # wide N, K with few rows: u's contraction ragged past 32 blocks
    (2048, 2048, 40, 64, 16.0),    # four 16-wide tiles over 32 column blocks
    (1024, 1024, 48, 128, 16.0),   # eight tiles (8 waves per workgroup)
    (264, 256, 2050, 16, 32.0),    # many row groups, ragged M
    (200, 192, 45, 5, 10.0),       # r % 8 != 0: B rows read element by element in u = G B
    (264, 320, 37, 13, 16.0),      # r % 8 != 0, N % 64 != 0
    (136, 128, 40, 100, 16.0),     # r % 8 != 0 with seven 16-wide tiles
    (4104, 256, 24, 16, 32.0),     # u over 65 column blocks (two rounds of four per wave), B as given
    (4104, 256, 24, 40, 16.0),     # same, B transposed first
    (520, 4096, 40, 16, 32.0),     # recomputed t over 64 column blocks
])
@pytest.mark.parametrize("recompute_t", [False, True])
def test_backward(lq, torch, N, K, M, r, alpha, recompute_t):
    L, W, X, A, B = make_layer(200 + M, N, K, M, r, alpha)
    G = syn.grad_out(L)
    qw = lq.QWeight.from_weight(dev(torch, W))
    Xd, Ad, Bd, Gd = (bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits),
                      bf16_dev(torch, G.bits))
    _, t = lq.qlora_forward(qw, Xd, Ad, Bd, alpha)
    gx, dA, dB = lq.qlora_backward(qw, Xd, Gd, Ad, Bd, alpha, t=None if recompute_t else t)
    Wd = oracle_wd(W)
    rX, rA, rB = layer.backward(Wd, X.f32, G.f32, A.f32, B.f32, alpha)
    assert layer.rel_frobenius(bf16_to_f32(gx), rX) <= BF16_TOL
    assert layer.rel_frobenius(host(dA), rA) <= F32_TOL
    assert layer.rel_frobenius(host(dB), rB) <= F32_TOL


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (True, True, False), (False, True, True), (True, False, True)])
def test_backward_output_subsets(lq, torch, need):
    """Any subset of (grad_X, dA, dB): each requested output matches the
    oracle and the others come back as None (dA alone moves the column-form
    job into the first slot of the merged launch)."""
    need_gx, need_dA, need_dB = need
    N, K, M, r, alpha = 264, 320, 70, 24, 8.0
    L, W, X, A, B = make_layer(900, N, K, M, r, alpha)
    G = syn.grad_out(L)
    qw = lq.QWeight.from_weight(dev(torch, W))
    Xd, Ad, Bd, Gd = (bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits),
                      bf16_dev(torch, G.bits))
    _, t = lq.qlora_forward(qw, Xd, Ad, Bd, alpha)
    gx, dA, dB = lq.qlora_backward(qw, Xd, Gd, Ad, Bd, alpha, t=t, need_grad_x=need_gx, need_dA=need_dA,
                                   need_dB=need_dB)
    rX, rA, rB = layer.backward(oracle_wd(W), X.f32, G.f32, A.f32, B.f32, alpha)
    assert (gx is not None) == need_gx and (dA is not None) == need_dA and (dB is not None) == need_dB
    if need_gx:
        assert layer.rel_frobenius(bf16_to_f32(gx), rX) <= BF16_TOL
    if need_dA:
        assert layer.rel_frobenius(host(dA), rA) <= F32_TOL
    if need_dB:
        assert layer.rel_frobenius(host(dB), rB) <= F32_TOL


def test_backward_grad_x_unit_probe(lq, torch):
    """G rows = e_n, B = 0 (so u = 0): grad_X[m, :] = W'[n_m, :] exactly."""
    rng = np.random.default_rng(4)
    N, K, M = 256, 384, 40
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ns = rng.integers(0, N, M)
    G = np.zeros((M, N), dtype=np.uint16)
    G[np.arange(M), ns] = 0x3F80
    X = syn.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    A = syn.to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32))
    B = np.zeros((N, 16), dtype=np.uint16)
    qw = lq.QWeight.from_weight(dev(torch, W))
    gx, dA, dB = lq.qlora_backward(qw, bf16_dev(torch, X), bf16_dev(torch, G), bf16_dev(torch, A),
                                   bf16_dev(torch, B), 32.0)
    Wd = oracle_wd(W)
    assert np.array_equal(bf16_to_f32(gx), Wd[ns])
    assert np.all(host(dA) == 0)


# ---------------------------------------------------------------------------
# codebook path
# ---------------------------------------------------------------------------
def codebook_case(seed, N, K):
    rng = np.random.default_rng(seed)
    sig = 0.02 * np.exp(0.3 * rng.standard_normal(N))
    W = (rng.standard_normal((N, K)) * sig[:, None]).astype(np.float32)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    L, T = lloyd.learn_codebooks(W, bits)
    return W, bits, L, T


def test_codebook_quantize_bit_exact(lq, torch):
    W, bits, L, T = codebook_case(1, 200, 384)
    codes, absmax, row_off = lq.quantize_codebook(dev(torch, W), dev(torch, bits), dev(torch, T))
    packed, c, _ = codebook.quantize(W, bits, T)
    assert np.array_equal(host(absmax), c)
    assert np.array_equal(host(row_off), codebook.row_offsets(bits, 384))
    assert np.array_equal(host(codes)[:packed.size], packed)


@pytest.mark.parametrize("dtype,offset", [("f32", 1), ("bf16", 0), ("bf16", 1), ("f16", 0), ("f16", 3)])
def test_codebook_quantize_half_and_unaligned(lq, torch, dtype, offset):
    """bf16 / f16 inputs (widened exactly) and base pointers off the vector
    alignment (element offset into a larger buffer); K not a multiple of 256."""
    W, bits, L, T = codebook_case(4, 72, 320)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    buf = torch.zeros(W.size + 8, dtype=tdt, device="cuda")
    Wd = buf[offset:offset + W.size].view(W.shape)
    Wd.copy_(dev(torch, W).to(tdt))
    W32 = host(Wd.float())
    codes, absmax, row_off = lq.quantize_codebook(Wd, dev(torch, bits), dev(torch, T))
    packed, c, _ = codebook.quantize(W32, bits, T)
    assert np.array_equal(host(absmax), c)
    assert np.array_equal(host(codes)[:packed.size], packed)


def test_codebook_nf4_cross_check(lq, torch):
    """4 bits with the NF4 thresholds/levels: dequant equals the NF4 path's."""
    rng = np.random.default_rng(2)
    N, K = 128, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bits = np.full(N, 4, dtype=np.uint8)
    T = np.tile(nf4.thresholds(), (N, 1)).astype(np.float32)
    Lv = np.tile(nf4.levels(), (N, 1)).astype(np.float32)
    qc = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv))
    qn = lq.QWeight.from_weight(dev(torch, W))
    assert np.array_equal(bf16_to_f32(lq.dequant(qc)), bf16_to_f32(lq.dequant(qn)))


@pytest.mark.parametrize("M", [64, 300])
def test_codebook_dequant_and_forward(lq, torch, M):
    N, K, r, alpha = 256, 512, 16, 32.0
    W, bits, Lv, T = codebook_case(3, N, K)
    qw = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv))
    packed, c, _ = codebook.quantize(W, bits, T)
    code8, s2, mu = dq.double_quant(c)
    cp = dq.dq_decode(code8, s2, mu)
    Wd = codebook.dequant(packed, bits, Lv, cp, N, K)
    assert np.array_equal(bf16_to_f32(lq.dequant(qw)).view(np.uint32), Wd.view(np.uint32))
    Ls = syn.small_layer(N, K, M, r, alpha, 300 + M)
    X, A, B = syn.activations(Ls), syn.lora_a(Ls), syn.lora_b(Ls)
    H, t = lq.qlora_forward(qw, bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits), alpha)
    Href, _ = layer.forward(Wd, X.f32, A.f32, B.f32, alpha)
    assert layer.rel_frobenius(bf16_to_f32(H), Href) <= BF16_TOL


def codebook_oracle_wd(W, bits, Lv, T):
    N, K = W.shape
    packed, c, _ = codebook.quantize(W, bits, T)
    code8, s2, mu = dq.double_quant(c)
    return codebook.dequant(packed, bits, Lv, dq.dq_decode(code8, s2, mu), N, K)


@pytest.mark.parametrize("N,K,M,r,alpha", [(256, 512, 300, 16, 32.0), (200, 320, 70, 64, 16.0)])
def test_codebook_forward_f32_and_backward(lq, torch, N, K, M, r, alpha):
    """Codebook weights through the full layer: forward (bf16 and float32 H)
    and backward (grad_X through the dequantized weight, dA, dB); N = 200
    leaves a partial last step of the backward's contraction."""
    W, bits, Lv, T = codebook_case(7 + M, N, K)
    qw = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv))
    Wd = codebook_oracle_wd(W, bits, Lv, T)
    Ls = syn.small_layer(N, K, M, r, alpha, 400 + M)
    X, A, B, G = syn.activations(Ls), syn.lora_a(Ls), syn.lora_b(Ls), syn.grad_out(Ls)
    Xd, Ad, Bd, Gd = (bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits),
                      bf16_dev(torch, G.bits))
    H, t = lq.qlora_forward(qw, Xd, Ad, Bd, alpha)
    H32, _ = lq.qlora_forward(qw, Xd, Ad, Bd, alpha, out_dtype=torch.float32)
    Href, tref = layer.forward(Wd, X.f32, A.f32, B.f32, alpha)
    assert layer.rel_frobenius(bf16_to_f32(H), Href) <= BF16_TOL
    assert layer.rel_frobenius(host(H32), Href) <= F32_TOL
    gx, dA, dB = lq.qlora_backward(qw, Xd, Gd, Ad, Bd, alpha, t=t)
    rX, rA, rB = layer.backward(Wd, X.f32, G.f32, A.f32, B.f32, alpha)
    assert layer.rel_frobenius(bf16_to_f32(gx), rX) <= BF16_TOL
    assert layer.rel_frobenius(host(dA), rA) <= F32_TOL
    assert layer.rel_frobenius(host(dB), rB) <= F32_TOL


def codebook_case_widths(seed, N, K, widths):
    """Like codebook_case with the widths given: an int (every row), or
    "mixed" (random rows of 1..4 bits, the widest differing between row
    groups)."""
    rng = np.random.default_rng(seed)
    sig = 0.02 * np.exp(0.3 * rng.standard_normal(N))
    W = (rng.standard_normal((N, K)) * sig[:, None]).astype(np.float32)
    if widths == "mixed":
        bits = rng.integers(1, 5, N).astype(np.uint8)
        bits[:16] = rng.integers(1, 3, 16)          # a row group of 1- and 2-bit rows
        bits[16:32] = rng.integers(1, 4, 16)        # one of at most 3 bits
    else:
        bits = np.full(N, widths, dtype=np.uint8)
    L, T = lloyd.learn_codebooks(W, bits)
    return W, bits, L, T


@pytest.mark.parametrize("N,K,M,widths,double", [
    (256, 512, 1, "mixed", True),
    (200, 1344, 4, "mixed", True),     # ragged N, K/64 = 21 (a half-empty last stage)
    (96, 4096, 16, "mixed", False),    # float32 constants
    (64, 256, 16, 1, True),
    (64, 320, 7, 2, True),
    (48, 640, 16, 3, False),
    (33, 2048, 3, 4, True),            # one row past two whole row groups
])
def test_codebook_decode_gemv(lq, torch, monkeypatch, N, K, M, widths, double):
    """The codebook decode kernel (M <= 16) against the oracle, in float32 and
    bfloat16 H, and against the GEMM path on the same inputs."""
    W, bits, Lv, T = codebook_case_widths(N + K + M, N, K, widths)
    qw = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv),
                                  double_quantize=double)
    packed, c, _ = codebook.quantize(W, bits, T)
    cp = dq.dq_decode(*dq.double_quant(c)) if double else c
    Wd = codebook.dequant(packed, bits, Lv, cp, N, K)
    Ls = syn.small_layer(N, K, M, 16, 32.0, 500 + N)
    X, A, B = syn.activations(Ls), syn.lora_a(Ls), syn.lora_b(Ls)
    args = (qw, bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits), 32.0)
    H32, _ = lq.qlora_forward(*args, out_dtype=torch.float32)
    H16, _ = lq.qlora_forward(*args)
    Href, _ = layer.forward(Wd, X.f32, A.f32, B.f32, 32.0)
    assert layer.rel_frobenius(host(H32), Href) <= F32_TOL
    assert layer.rel_frobenius(bf16_to_f32(H16), Href) <= BF16_TOL
    monkeypatch.setenv("LQ_FORCE_PATH", "gemm")
    Hg, _ = lq.qlora_forward(*args, out_dtype=torch.float32)
    assert layer.rel_frobenius(host(H32), host(Hg)) <= F32_TOL


def test_codebook_decode_gemv_unit_columns(lq, torch):
    """X rows = unit vectors e_k, B = 0: H[m, n] = W'[n, k_m] exactly, so every
    code the decode kernel reads (each bit-plane, both halves of a block,
    every row width, rows past a whole row group) is checked bit for bit."""
    N, K, M = 80, 1408, 16
    W, bits, Lv, T = codebook_case_widths(77, N, K, "mixed")
    qw = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv))
    Wd = codebook_oracle_wd(W, bits, Lv, T)
    rng = np.random.default_rng(78)
    A = syn.to_bf16_bits((rng.standard_normal((16, K)) * 0.02).astype(np.float32))
    B = np.zeros((N, 16), dtype=np.uint16)
    ks = np.concatenate([np.arange(0, 64, 4), rng.permutation(K)[:48]])
    for c0 in range(0, ks.size, M):
        kk = ks[c0:c0 + M]
        X = np.zeros((M, K), dtype=np.uint16)
        X[np.arange(M), kk] = 0x3F80
        H, _ = lq.qlora_forward(qw, bf16_dev(torch, X), bf16_dev(torch, A), bf16_dev(torch, B), 32.0,
                                out_dtype=torch.float32)
        assert np.array_equal(host(H), Wd[:, kk].T)


def test_codebook_grad_x_unit_probe(lq, torch):
    """G rows = e_n, B = 0: grad_X[m, :] = W'[n_m, :] exactly (the
    transposed copy of the dequantized codebook weight)."""
    rng = np.random.default_rng(6)
    N, K, M = 136, 384, 40
    W, bits, Lv, T = codebook_case(9, N, K)
    ns = rng.integers(0, N, M)
    G = np.zeros((M, N), dtype=np.uint16)
    G[np.arange(M), ns] = 0x3F80
    X = syn.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    A = syn.to_bf16_bits(rng.standard_normal((16, K)).astype(np.float32))
    B = np.zeros((N, 16), dtype=np.uint16)
    qw = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv))
    gx, dA, dB = lq.qlora_backward(qw, bf16_dev(torch, X), bf16_dev(torch, G), bf16_dev(torch, A),
                                   bf16_dev(torch, B), 32.0)
    Wd = codebook_oracle_wd(W, bits, Lv, T)
    assert np.array_equal(bf16_to_f32(gx), Wd[ns])


# ---------------------------------------------------------------------------
# AQLoRA profiling pass
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(64, 64), (192, 320), (1000, 128), (37, 1024)])
def test_profile_matches_oracle(lq, torch, shape):
    """eps to float64 summation-order rounding; the small-weight count exactly."""
    rng = np.random.default_rng(shape[0] + 3 * shape[1])
    W = edge_weight(rng, *shape) if shape[0] * shape[1] >= 64 * 64 else \
        (rng.standard_normal(shape) * 0.02).astype(np.float32)
    stats = host(lq.profile_nf4(dev(torch, W)))
    eps, s = nf4.profile(W)
    assert stats[0] == pytest.approx(eps, rel=1e-10, abs=1e-300)
    assert round(stats[1] * W.size) == round(s * W.size)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_profile_half_inputs(lq, torch, dtype):
    rng = np.random.default_rng(8)
    W32 = (rng.standard_normal((96, 256)) * 0.02).astype(np.float32)
    t = torch.from_numpy(W32).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    Wexact = t.float().numpy()
    stats = host(lq.profile_nf4(t.cuda()))
    eps, s = nf4.profile(Wexact)
    assert stats[0] == pytest.approx(eps, rel=1e-10)
    assert round(stats[1] * W32.size) == round(s * W32.size)
