"""GPU parity at the benchmarked sizes, on sampled outputs.

The workloads run through the same entry points and launch configurations as
the benchmark: q_proj (4096 x 4096, 2048 tokens, r = 16), the MLP pair
(11008 x 4096 and 4096 x 11008, 4096 tokens, r = 64), the decode GEMV
(28672 x 8192 at 1, 4 and 16 tokens) and the 1.75-bit per-channel codebook
layer (4096 x 4096, 2048 tokens). The whole weight is quantized on the GPU;
the oracle recomputes what it can one piece at a time:
  * block constants of every block (a plain reduction), and from them the
    double quantization of the whole tensor (bit-exact);
  * codes and dequantized rows for sampled rows, and whole 64-column blocks
    for sampled columns (blocks are independent, bit-exact);
  * H on sampled (token, output) pairs, grad_X on sampled (token, input)
    pairs, dA and dB in full (relative Frobenius error on the sample).
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


def bf16_bits(t):
    import torch
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def bf16_to_f32(t):
    return (bf16_bits(t).astype(np.uint32) << 16).view(np.float32)


def sample(rng, n, k):
    """k sorted distinct indices in [0, n) including both ends."""
    idx = rng.choice(n, size=min(k, n), replace=False)
    idx[:2] = [0, n - 1]
    return np.unique(idx)


def oracle_constants(W):
    """Oracle block constants of the whole weight and their double quantization."""
    c = nf4.block_absmax(W)
    code8, s2, mu = dq.double_quant(c)
    return c, (code8, s2, mu), dq.dq_decode(code8, s2, mu)


def oracle_rows(W, rows, cp):
    """Oracle codes and bf16 weights of whole rows (blocks run along rows)."""
    N, K = W.shape
    packed, c = nf4.quantize(W[rows])
    cpr = cp.reshape(N, K // 64)[rows].reshape(-1)
    return packed.reshape(len(rows), K // 2), c, nf4.dequant(packed, cpr, (len(rows), K))


def oracle_col_blocks(W, blocks, cp):
    """Oracle bf16 weights of whole 64-column blocks (all rows)."""
    N, K = W.shape
    cols = (64 * blocks[:, None] + np.arange(64)[None, :]).reshape(-1)
    packed, _ = nf4.quantize(np.ascontiguousarray(W[:, cols]))
    cpc = cp.reshape(N, K // 64)[:, blocks].reshape(-1)
    return cols, nf4.dequant(packed, cpc, (N, cols.size))


def check_profile(lq, torch, W):
    """AQLoRA profiling pass over the whole layer against the oracle."""
    stats = host(lq.profile_nf4(dev(torch, W)))
    eps, s = nf4.profile(W)
    assert stats[0] == pytest.approx(eps, rel=1e-9)
    assert round(stats[1] * W.size) == round(s * W.size)


def check_codec(lq, torch, W, qw, rows, cp_ref, dqp_ref, c_ref):
    N, K = W.shape
    code8, s2, mu = dqp_ref
    # double quantization of the whole tensor, bit-exact
    assert np.array_equal(host(qw.absmax_q), code8)
    assert np.array_equal(host(qw.dq_scale).view(np.uint32), s2.view(np.uint32))
    assert host(qw.dq_mean).view(np.uint32)[0] == np.float32(mu).view(np.uint32)
    # codes of sampled rows, bit-exact
    pk, c_rows, wd_rows = oracle_rows(W, rows, cp_ref)
    codes = host(qw.codes).reshape(N, K // 2)
    assert np.array_equal(codes[rows], pk)
    # dequantized rows, bit-exact
    Wd = lq.dequant(qw)
    got = bf16_to_f32(Wd[dev(torch, rows)])
    assert np.array_equal(got.view(np.uint32), wd_rows.view(np.uint32))
    return wd_rows


def quantize_on_gpu(lq, torch, W):
    """Quantize on the GPU keeping float32 absmax too (for the bit-exact check)."""
    Wg = dev(torch, W)
    codes, absmax = lq.quantize_nf4(Wg)
    aq, s2, mu = lq.double_quant(absmax)
    del Wg
    N, K = W.shape
    return codes, absmax, lq.QWeight(N, K, codes, absmax_q=aq, dq_scale=s2, dq_mean=mu)


@pytest.mark.parametrize("name", ["q_proj", "mlp_up", "mlp_down"])
def test_prefill_layer_full_size(lq, torch, name):
    L = syn.LAYERS[name]
    N, K, M, r, alpha = L.N, L.K, L.M, L.r, L.alpha
    rng = np.random.default_rng(L.workload_id)
    W = syn.weight(L)
    c_ref, dqp, cp = oracle_constants(W)
    codes, absmax, qw = quantize_on_gpu(lq, torch, W)
    assert np.array_equal(host(absmax).view(np.uint32), c_ref.view(np.uint32))
    rows = sample(rng, N, 192)
    wd_rows = check_codec(lq, torch, W, qw, rows, cp, dqp, c_ref)
    check_profile(lq, torch, W)

    X, A, B, G = syn.activations(L), syn.lora_a(L), syn.lora_b(L), syn.grad_out(L)
    Xd, Ad, Bd, Gd = (bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits),
                      bf16_dev(torch, G.bits))
    # forward: H on sampled tokens x sampled outputs (the rows whose W' the oracle has)
    H, t = lq.qlora_forward(qw, Xd, Ad, Bd, alpha)
    ms = sample(rng, M, 96)
    Href, tref = layer.forward(wd_rows, X.f32[ms], A.f32, B.f32[rows], alpha, r)
    assert layer.rel_frobenius(host(t)[ms], tref) <= 1e-5
    assert layer.rel_frobenius(bf16_to_f32(H)[np.ix_(ms, rows)], Href) <= BF16_TOL
    H32 = lq.dequant_gemm(qw, Xd, t, Bd, alpha, out_dtype=torch.float32)
    assert layer.rel_frobenius(host(H32)[np.ix_(ms, rows)], Href) <= F32_TOL
    del H, H32

    # backward: dA, dB in full; grad_X on sampled tokens x whole sampled column blocks
    gx, dA, dB = lq.qlora_backward(qw, Xd, Gd, Ad, Bd, alpha, t=t)
    s = alpha / r
    X64, G64, A64, B64 = (X.f32.astype(np.float64), G.f32.astype(np.float64),
                          A.f32.astype(np.float64), B.f32.astype(np.float64))
    t64 = X64 @ A64.T
    u64 = G64 @ B64
    assert layer.rel_frobenius(host(dB), s * (G64.T @ t64)) <= F32_TOL
    assert layer.rel_frobenius(host(dA), s * (u64.T @ X64)) <= F32_TOL
    blocks = np.unique(rng.choice(K // 64, size=4, replace=False))
    cols, wd_cols = oracle_col_blocks(W, blocks, cp)
    gref = G64[ms] @ wd_cols.astype(np.float64) + s * (u64[ms] @ A64[:, cols])
    assert layer.rel_frobenius(bf16_to_f32(gx)[np.ix_(ms, cols)], gref) <= BF16_TOL


@pytest.mark.parametrize("direction", ["forward", "backward", "backward_ragged"])
def test_split_tail_tiles(lq, torch, direction):
    """264 output tiles of 256 x 128 (33 per XCD: one full round of 32 and one
    more), so the last tile of every XCD runs as two halves of the
    contraction whose partial sums a second kernel adds; every output column
    on 64 sampled tokens against the oracle, bf16 and float32 forward
    outputs and grad_X (also with a contraction whose last step is partial,
    which falls in the second half)."""
    M, r, alpha = 512, 16, 32.0
    # backward_ragged: a contraction of 1000 rows (16 steps, the last one partial)
    N, K = {"forward": (132 * 128, 1024), "backward": (1024, 132 * 128),
            "backward_ragged": (1000, 132 * 128)}[direction]
    L = syn.small_layer(N, K, M, r, alpha, seed={"forward": 901, "backward": 902, "backward_ragged": 904}[direction])
    W = syn.weight(L)
    rng = np.random.default_rng(L.workload_id)
    c_ref, dqp, cp = oracle_constants(W)
    codes, absmax, qw = quantize_on_gpu(lq, torch, W)
    X, A, B, G = syn.activations(L), syn.lora_a(L), syn.lora_b(L), syn.grad_out(L)
    Xd, Ad, Bd, Gd = (bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits),
                      bf16_dev(torch, G.bits))
    ms = np.unique(np.concatenate([sample(rng, 256, 32), 256 + sample(rng, 256, 32)]))   # both M-tiles
    s = alpha / r
    if direction == "forward":
        _, _, wd = oracle_rows(W, np.arange(N), cp)           # every output row of W'
        H, t = lq.qlora_forward(qw, Xd, Ad, Bd, alpha)
        Href, _ = layer.forward(wd, X.f32[ms], A.f32, B.f32, alpha, r)
        assert layer.rel_frobenius(bf16_to_f32(H)[ms], Href) <= BF16_TOL
        H32 = lq.dequant_gemm(qw, Xd, t, Bd, alpha, out_dtype=torch.float32)
        assert layer.rel_frobenius(host(H32)[ms], Href) <= F32_TOL
    else:
        cols, wd = oracle_col_blocks(W, np.arange(K // 64), cp)   # the whole W' by columns
        assert np.array_equal(cols, np.arange(K))
        t = lq.lora_down(Xd, Ad)
        gx, _, _ = lq.qlora_backward(qw, Xd, Gd, Ad, Bd, alpha, t=t, need_dA=False, need_dB=False)
        u64 = G.f32.astype(np.float64) @ B.f32.astype(np.float64)
        gref = G.f32[ms].astype(np.float64) @ wd.astype(np.float64) + s * (u64[ms] @ A.f32.astype(np.float64))
        assert layer.rel_frobenius(bf16_to_f32(gx)[ms], gref) <= BF16_TOL


def test_split_tail_tiles_codebook(lq, torch):
    """The same 264-tile forward over a per-channel codebook weight (random
    widths, levels and midpoint thresholds per row): the GEMM reads the
    dequantized weight from the workspace, and the split tiles' partial sums
    sit behind it in the same workspace."""
    M, r, alpha = 512, 16, 32.0
    N, K = 132 * 128, 1024
    L = syn.small_layer(N, K, M, r, alpha, seed=903)
    W = syn.weight(L)
    rng = np.random.default_rng(L.workload_id)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    Lv = np.zeros((N, 16), np.float32)
    T = np.full((N, 15), 3.0, np.float32)
    for i, b in enumerate(bits):
        n = 1 << int(b)
        Lv[i, :n] = np.sort(rng.uniform(-1.0, 1.0, n)).astype(np.float32)
        T[i, :n - 1] = nf4.midpoint_thresholds(Lv[i, :n])
    qw = lq.QWeight.from_codebook(dev(torch, W), dev(torch, bits), dev(torch, T), dev(torch, Lv))
    _, _, cp = oracle_constants(W)
    packed, _, _ = codebook.quantize(W, bits, T)
    wd = codebook.dequant(packed, bits, Lv, cp, N, K)
    X, A, B = syn.activations(L), syn.lora_a(L), syn.lora_b(L)
    H, _ = lq.qlora_forward(qw, bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits), alpha)
    ms = np.unique(np.concatenate([sample(rng, 256, 32), 256 + sample(rng, 256, 32)]))
    Href, _ = layer.forward(wd, X.f32[ms], A.f32, B.f32, alpha, r)
    assert layer.rel_frobenius(bf16_to_f32(H)[ms], Href) <= BF16_TOL


def test_q_proj_forward_f32_elementwise_bound(lq, torch):
    """q_proj forward with float32 H (4096 x 4096, 2048 tokens, r = 16) on
    sampled (token, output) pairs, each element within a worst-case rounding
    bound of the exact result from the bf16 inputs and the dequantized weight
    (QLoRA page, eq. 5: H = X W'^T + s X A^T B^T). The MFMAs multiply bf16
    pairs exactly and add in float32, so a K-term sum errs by at most
    (K + c) u sum |x w'| (u = 2^-24) in any order; the LoRA term goes through
    t = X A^T (same bound, r sums of K terms) and the hi/lo bfloat16 split of
    s t (relative error below 2^-16), then a 2r-term sum."""
    L = syn.LAYERS["q_proj"]
    N, K, M, r, alpha = L.N, L.K, L.M, L.r, L.alpha
    s = alpha / r
    u = 2.0 ** -24
    rng = np.random.default_rng(77)
    W = syn.weight(L)
    _, _, cp = oracle_constants(W)
    _, _, qw = quantize_on_gpu(lq, torch, W)
    X, A, B = syn.activations(L), syn.lora_a(L), syn.lora_b(L)
    H, t = lq.qlora_forward(qw, bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits), alpha,
                            out_dtype=torch.float32)
    rows = sample(rng, N, 64)
    ms = sample(rng, M, 64)
    _, _, wd = oracle_rows(W, rows, cp)
    x = X.f32[ms].astype(np.float64)
    w = wd.astype(np.float64)
    a = A.f32.astype(np.float64)
    b = B.f32[rows].astype(np.float64)
    t_ex = x @ a.T                                      # [m, r]
    h_ex = x @ w.T + s * (t_ex @ b.T)
    sxw = np.abs(x) @ np.abs(w).T
    sxa = np.abs(x) @ np.abs(a).T                       # [m, r]
    dt = (K + 4) * u * sxa + 2.0 ** -16 * np.abs(t_ex) * (1 + (K + 4) * u)
    lora_abs = np.abs(t_ex) @ np.abs(b).T
    bound = (K + 2 * r + 8) * u * (sxw + abs(s) * (lora_abs + dt @ np.abs(b).T)) + abs(s) * (dt @ np.abs(b).T)
    err = np.abs(host(H)[np.ix_(ms, rows)].astype(np.float64) - h_ex)
    assert np.all(err <= bound), float(np.max(err / bound))
    # the bound is loose by design (worst case); the typical error is far below it
    assert float(np.median(err / bound)) < 0.05


@pytest.fixture(scope="module")
def decode_case(lq, torch):
    L = syn.LAYERS["decode"]
    W = syn.weight(L)
    c_ref, dqp, cp = oracle_constants(W)
    codes, absmax, qw = quantize_on_gpu(lq, torch, W)
    rows = sample(np.random.default_rng(4), L.N, 256)
    return L, W, c_ref, dqp, cp, absmax, qw, rows


def test_decode_codec_full_size(lq, torch, decode_case):
    L, W, c_ref, dqp, cp, absmax, qw, rows = decode_case
    assert np.array_equal(host(absmax).view(np.uint32), c_ref.view(np.uint32))
    check_codec(lq, torch, W, qw, rows, cp, dqp, c_ref)
    check_profile(lq, torch, W)


@pytest.mark.parametrize("M", list(syn.DECODE_TOKENS))
def test_decode_gemv_full_size(lq, torch, decode_case, M):
    L, W, c_ref, dqp, cp, absmax, qw, rows = decode_case
    _, _, wd_rows = oracle_rows(W, rows, cp)
    X, A, B = syn.activations(L, M), syn.lora_a(L), syn.lora_b(L)
    Xd, Ad, Bd = bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits)
    t = lq.lora_down(Xd, Ad)
    H = lq.dequant_gemm(qw, Xd, t, Bd, L.alpha)
    H32 = lq.dequant_gemm(qw, Xd, t, Bd, L.alpha, out_dtype=torch.float32)
    Href, tref = layer.forward(wd_rows, X.f32, A.f32, B.f32[rows], L.alpha, L.r)
    assert layer.rel_frobenius(host(t), tref) <= 1e-5
    assert layer.rel_frobenius(bf16_to_f32(H)[:, rows], Href) <= BF16_TOL
    assert layer.rel_frobenius(host(H32)[:, rows], Href) <= F32_TOL


@pytest.mark.parametrize("M", list(syn.DECODE_TOKENS))
def test_decode_forward_full_size(lq, torch, decode_case, M):
    """The whole forward at decode sizes (one launch: t = X A^T is formed
    inside the GEMV): t in full and sampled rows of H."""
    L, W, c_ref, dqp, cp, absmax, qw, rows = decode_case
    _, _, wd_rows = oracle_rows(W, rows, cp)
    X, A, B = syn.activations(L, M), syn.lora_a(L), syn.lora_b(L)
    Xd, Ad, Bd = bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits)
    H, t = lq.qlora_forward(qw, Xd, Ad, Bd, L.alpha)
    H32, t32 = lq.qlora_forward(qw, Xd, Ad, Bd, L.alpha, out_dtype=torch.float32)
    Href, tref = layer.forward(wd_rows, X.f32, A.f32, B.f32[rows], L.alpha, L.r)
    assert layer.rel_frobenius(host(t), tref) <= 1e-5
    assert torch.equal(t, t32)
    assert layer.rel_frobenius(bf16_to_f32(H)[:, rows], Href) <= BF16_TOL
    assert layer.rel_frobenius(host(H32)[:, rows], Href) <= F32_TOL


def test_codebook_layer_full_size(lq, torch):
    """1.75-bit per-channel layer with its tables learned on the GPU by the
    weighted Lloyd-Max learner (checked against the oracle's learner on
    sampled rows), then quantized, dequantized and run forward."""
    L = syn.LAYERS["lowra"]
    N, K, M, r, alpha = L.N, L.K, L.M, L.r, L.alpha
    W = syn.weight(L)
    bits = syn.lowra_row_bits(L)
    Wdev = dev(torch, W)
    Lg, Tg, itg = lq.lloyd_codebooks(Wdev, dev(torch, bits))
    Lv, T, it = host(Lg), host(Tg), host(itg)
    rng = np.random.default_rng(5)
    rows = sample(rng, N, 192)
    Lr, Tr, itr = lloyd.learn_codebooks(W[rows], bits[rows], return_iters=True)
    assert np.array_equal(it[rows], itr)
    Lo = Lv[rows]
    assert np.all((Lo == Lr) | (Lo == np.nextafter(Lr, np.float32(np.inf)))
                  | (Lo == np.nextafter(Lr, np.float32(-np.inf))))
    assert np.mean(np.all(Lo == Lr, axis=1)) >= 0.99
    for i in rows:
        n = 1 << int(bits[i])
        assert np.array_equal(T[i, :n - 1].view(np.uint32),
                              nf4.midpoint_thresholds(Lv[i, :n]).view(np.uint32))
    qw = lq.QWeight.from_codebook(Wdev, dev(torch, bits), Tg, Lg)
    c_ref, (code8, s2, mu), cp = oracle_constants(W)
    assert np.array_equal(host(qw.absmax_q), code8)
    assert np.array_equal(host(qw.dq_scale).view(np.uint32), s2.view(np.uint32))

    packed, _, _ = codebook.quantize(W[rows], bits[rows], T[rows])
    off_full = codebook.row_offsets(bits, K)
    off_sub = codebook.row_offsets(bits[rows], K)
    got = host(qw.codes)
    for j, i in enumerate(rows):
        assert np.array_equal(got[off_full[i]:off_full[i + 1]], packed[off_sub[j]:off_sub[j + 1]])
    cpr = cp.reshape(N, K // 64)[rows].reshape(-1)
    wd_rows = codebook.dequant(packed, bits[rows], Lv[rows], cpr, len(rows), K)
    Wd = lq.dequant(qw)
    assert np.array_equal(bf16_to_f32(Wd[dev(torch, rows)]).view(np.uint32), wd_rows.view(np.uint32))

    X, A, B = syn.activations(L), syn.lora_a(L), syn.lora_b(L)
    H, t = lq.qlora_forward(qw, bf16_dev(torch, X.bits), bf16_dev(torch, A.bits), bf16_dev(torch, B.bits), alpha)
    ms = sample(rng, M, 96)
    Href, _ = layer.forward(wd_rows, X.f32[ms], A.f32, B.f32[rows], alpha, r)
    assert layer.rel_frobenius(bf16_to_f32(H)[np.ix_(ms, rows)], Href) <= BF16_TOL


def test_loftq_full_size(lq, torch):
    """LoftQ-style initialisation of the q_proj adapter (4096 x 4096, r = 16,
    l = 32, 8 power steps, 5 alternations), in the configuration bench.py
    times. Step 1 quantizes W itself (bit-exact on sampled rows against the
    oracle with the whole tensor's double quantization); its residual is
    bit-exact on the same rows; the rank-16 SVD of the step-1 residual is
    checked against the exact singular values of that residual (Ritz values
    never above them and within 3% below: 8 power steps on a 2r-column
    sketch separate this residual's flat spectrum that far; error left within
    2e-3 of the optimum); five steps leave less error than one."""
    L = syn.LAYERS["q_proj"]
    N, K, r, l, q = L.N, L.K, L.r, 2 * L.r, 8
    W = syn.weight(L)
    Wd_, Om = dev(torch, W), dev(torch, np.random.default_rng(1).standard_normal((K, l)).astype(np.float32))
    qw1, B1, A1, s1, ob1 = lq.loftq_init(Wd_, r, Om, steps=1, power_iters=q)
    c_ref, (code8, s2, mu), cp = oracle_constants(W)
    assert np.array_equal(host(qw1.absmax_f32), c_ref)
    assert np.array_equal(host(qw1.absmax_q), code8)
    rng = np.random.default_rng(11)
    rows = sample(rng, N, 96)
    packed_rows, _, wd_rows = oracle_rows(W, rows, cp)
    got = host(qw1.codes).reshape(N, K // 2)
    assert np.array_equal(got[rows], packed_rows)
    R1 = host(lq.residual(Wd_, lq.dequant(qw1)))
    assert np.array_equal(R1[rows].view(np.uint32), (W[rows] - wd_rows).view(np.uint32))
    so = np.linalg.svd(R1.astype(np.float64), compute_uv=False)
    s = host(s1)
    assert np.all(s <= so[:r] * (1 + 1e-5)) and np.all(s >= 0.97 * so[:r])
    total = float(np.sum(so ** 2))
    opt = total - float(np.sum(so[:r] ** 2))
    assert opt <= host(ob1)[0] <= opt * (1 + 2e-3)
    qw5, B5, A5, s5, ob5 = lq.loftq_init(Wd_, r, Om, steps=5, power_iters=q)
    o5 = host(ob5)
    assert o5[0] == host(ob1)[0]
    assert o5[-1] < o5[0]


def test_loraquant_full_size(lq, torch):
    """LoRAQuant-style quantization of the MLP-up adapter (B 11008 x 64,
    A 64 x 4096, bf16 values), as bench.py times it: factors and singular
    values against the oracle's SVD of B A, the component count from the same
    float32 singular values, each component's learned codebook within one
    float32 ulp of the oracle learner's on the GPU's factors, and the codes
    bit-exact given the GPU's tables."""
    from oracle import loraquant
    L = syn.LAYERS["mlp_up"]
    A = syn.lora_a(L).f32
    B = syn.lora_b(L).f32
    q = lq.loraquant(dev(torch, B), dev(torch, A), rho=0.9, bits_hi=3, bits_lo=1)
    r, N, K = L.r, L.N, L.K
    Ap = host(q.Ap).reshape(r, K)
    Bp = host(q.Bpt).reshape(r, N).T
    sig = host(q.sigma)
    Bo, Ao, so = loraquant.reparam(B, A)
    assert np.max(np.abs(sig - so) / so) <= 1e-5
    assert np.max(np.abs(Ap - Ao)) <= 1e-4 * np.max(np.abs(Ao))
    h = int(host(q.h)[0])
    assert h == loraquant.choose_h(sig, 0.9)
    bits = loraquant.component_bits(r, h, 3, 1)
    qo = loraquant.quantize(Bp, Ap, bits)
    for side, X, codes, absmax, lv, th in (
            ("A", Ap, q.codes_a, q.absmax_a, q.levels_a, q.thresholds_a),
            ("B", np.ascontiguousarray(Bp.T), q.codes_b, q.absmax_b, q.levels_b, q.thresholds_b)):
        Lg, T = host(lv).reshape(r, 16), host(th).reshape(r, 15)
        Lr = qo[side]["levels"]
        near = (Lg == Lr) | (Lg == np.nextafter(Lr, np.float32(np.inf))) | (Lg == np.nextafter(Lr, np.float32(-np.inf)))
        assert np.all(near), side
        packed, c, _ = codebook.quantize(X, bits, T)
        assert np.array_equal(host(absmax), c)
        assert np.array_equal(host(codes)[:packed.size], packed)
