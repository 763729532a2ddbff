"""The LQ_DEBUG build on the GPU: same results as the release build on valid
input, the device flag word for precondition violations that kernels can
run through safely (non-finite weights, non-increasing thresholds), and the
host check that refuses an inconsistent codebook row layout before any
launch (LowRA page, section 3: per-channel precision and custom thresholds)."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lq():
    import quantized_lora_fine_lq_amd as mod
    return mod


@pytest.fixture(scope="module")
def dbg(lq):
    return lq.load_debug_library()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def flags(dbg, clear=True):
    v = ctypes.c_uint32(0)
    assert dbg.lq_debug_flags(ctypes.byref(v), 1 if clear else 0) == 0
    return v.value


def stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def codebook_inputs(torch, lq, N=96, K=256, seed=5):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bits = rng.integers(1, 5, N).astype(np.uint8)
    T = np.full((N, 15), 3.0, dtype=np.float32)
    for i, b in enumerate(bits):
        T[i, :(1 << b) - 1] = np.sort(rng.uniform(-0.95, 0.95, (1 << b) - 1)).astype(np.float32)
    off = np.array(lq.row_offsets(bits.tolist(), K), dtype=np.int64)
    return W, bits, T, off


def run_codebook(torch, L, W, bits, T, off):
    N, K = W.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    Wd, bd, Td, od = d(W), d(bits), d(T), d(off)
    codes = torch.zeros(int(off[-1]), dtype=torch.uint8, device="cuda")
    am = torch.zeros(N * K // 64, dtype=torch.float32, device="cuda")
    st = L.lq_quantize_codebook(P(Wd), 0, N, K, 64, P(bd), P(od), P(Td), P(codes), P(am), stream(torch))
    torch.cuda.synchronize()
    return st, codes.cpu().numpy(), am.cpu().numpy()


def test_debug_codebook_matches_release_and_flags_clean(lq, dbg, torch):
    W, bits, T, off = codebook_inputs(torch, lq)
    flags(dbg)
    st_r, c_r, a_r = run_codebook(torch, lq.lib, W, bits, T, off)
    st_d, c_d, a_d = run_codebook(torch, dbg, W, bits, T, off)
    assert st_r == 0 and st_d == 0
    assert np.array_equal(c_r, c_d) and np.array_equal(a_r, a_d)
    assert flags(dbg) == 0


def test_debug_flags_non_increasing_thresholds(lq, dbg, torch):
    W, bits, T, off = codebook_inputs(torch, lq, seed=6)
    i = int(np.nonzero(bits >= 2)[0][0])
    T[i, 1] = T[i, 0]            # a tie: not strictly increasing
    flags(dbg)
    st, _, _ = run_codebook(torch, dbg, W, bits, T, off)
    assert st == 0
    assert flags(dbg) & lq.LQ_DBG_THRESHOLDS
    assert flags(dbg) == 0       # cleared by the previous read


def test_debug_flags_non_finite_weight(lq, dbg, torch):
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    W[3, 17] = np.nan
    Wd = torch.from_numpy(W).cuda()
    codes = torch.empty(64 * 128, dtype=torch.uint8, device="cuda")
    am = torch.empty(64 * 4, dtype=torch.float32, device="cuda")
    flags(dbg)
    assert dbg.lq_quantize_nf4(P(Wd), 0, 64, 256, 64, P(codes), P(am), stream(torch)) == 0
    assert flags(dbg) & lq.LQ_DBG_NONFINITE
    W[3, 17] = 0.5
    Wd = torch.from_numpy(W).cuda()
    assert dbg.lq_quantize_nf4(P(Wd), 0, 64, 256, 64, P(codes), P(am), stream(torch)) == 0
    assert flags(dbg) == 0


def test_debug_refuses_bad_row_layout(lq, dbg, torch):
    W, bits, T, off = codebook_inputs(torch, lq, seed=8)
    bad = off.copy()
    bad[5:] += 8                 # row 4 claims 8 bytes more than K*b/8
    st, _, _ = run_codebook(torch, dbg, W, bits, T, bad)
    assert st == lq.LQ_ERR_ARG
    b2 = bits.copy()
    b2[0] = 6                    # a width outside 1..4
    st, _, _ = run_codebook(torch, dbg, W, b2, T, off)
    assert st == lq.LQ_ERR_ARG
    # the same check guards the dequantization of a codebook weight
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    N, K = W.shape
    lv = d(np.tile(np.linspace(-1, 1, 16, dtype=np.float32), (N, 1)))
    # sized for the bad offsets too, so that every access stays in bounds
    codes = torch.zeros(int(bad[-1]) + 256, dtype=torch.uint8, device="cuda")
    am = torch.ones(N * K // 64, dtype=torch.float32, device="cuda")
    bd, od = d(bits), d(bad)
    w = lq.lq_qweight(format=1, blocksize=64, N=N, K=K, codes=codes.data_ptr(), absmax=am.data_ptr(),
                      absmax_q=None, dq_scale=None, dq_mean=None, dq_blocksize=256, reserved0=0,
                      row_bits=bd.data_ptr(), row_offset=od.data_ptr(), levels=lv.data_ptr())
    out = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    assert dbg.lq_dequant(ctypes.byref(w), P(out), stream(torch)) == lq.LQ_ERR_ARG


def test_debug_layer_matches_release(lq, dbg, torch):
    """Forward and backward through the debug build (launch-shape asserts on)
    equal the release build's bit for bit."""
    rng = np.random.default_rng(9)
    N, K, M, r = 192, 320, 40, 16
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).cuda()
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16)
    X, A, B, G = (bf(rng.standard_normal((M, K))), bf(rng.standard_normal((r, K)) * 0.02),
                  bf(rng.standard_normal((N, r)) * 0.02), bf(rng.standard_normal((M, N))))
    qw = lq.QWeight.from_weight(W)
    outs = []
    for L in (lq.lib, dbg):
        H = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        t = torch.empty(M, r, dtype=torch.float32, device="cuda")
        fws = L.lq_forward_workspace(qw.ref(), M, r)
        ws = torch.empty(fws, dtype=torch.uint8, device="cuda")
        assert L.lq_qlora_forward(qw.ref(), P(X), M, P(A), P(B), r, 32.0, P(H), 1, P(t), P(ws), fws,
                                  stream(torch)) == 0
        gx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        dA = torch.empty(r, K, dtype=torch.float32, device="cuda")
        dB = torch.empty(N, r, dtype=torch.float32, device="cuda")
        bws = L.lq_backward_workspace(qw.ref(), M, r)
        wsb = torch.empty(bws, dtype=torch.uint8, device="cuda")
        assert L.lq_qlora_backward(qw.ref(), P(X), P(G), M, P(A), P(B), r, 32.0, P(t), P(gx), P(dA), P(dB),
                                   P(wsb), bws, stream(torch)) == 0
        torch.cuda.synchronize()
        outs.append([x.view(torch.int16).cpu().numpy() if x.dtype == torch.bfloat16 else x.cpu().numpy()
                     for x in (H, t, gx, dA, dB)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    assert flags(dbg) == 0
