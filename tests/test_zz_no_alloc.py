"""The no-allocation backward (scratch in a library-owned device array)
against lq_qlora_backward with a caller workspace: identical kernels, so the
outputs must be identical bit for bit. Calls run back to back, each smaller
than the one before, so a call that read scratch left over from the previous
one would show."""
import ctypes

import numpy as np
import pytest

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


def P(t):
    return ctypes.c_void_p(None) if t is None else ctypes.c_void_p(t.data_ptr())


def layer_inputs(torch, seed, N, K, M, r):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).cuda().to(torch.bfloat16)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).cuda()
    X, G = bf(rng.standard_normal((M, K))), bf(rng.standard_normal((M, N)))
    A, B = bf(rng.standard_normal((r, K)) * 0.02), bf(rng.standard_normal((N, r)) * 0.02)
    t = torch.from_numpy((rng.standard_normal((M, r))).astype(np.float32)).cuda()
    return W, X, G, A, B, t


def both(lq, torch, qw, X, G, A, B, t, r, alpha, need=(True, True, True)):
    """(workspace entry point outputs, no-allocation outputs) as host arrays."""
    M, N, K = G.shape[0], qw.N, qw.K
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = []
    for noalloc in (False, True):
        gx = torch.full((M, K), 7.0, dtype=torch.bfloat16, device="cuda") if need[0] else None
        dA = torch.full((r, K), 7.0, dtype=torch.float32, device="cuda") if need[1] else None
        dB = torch.full((N, r), 7.0, dtype=torch.float32, device="cuda") if need[2] else None
        if noalloc:
            assert lq.lib.lq_qlora_backward_noalloc_bytes(qw.ref(), M, r) <= lq.LQ_NOALLOC_SCRATCH_BYTES
            st = lq.lib.lq_qlora_backward_noalloc(qw.ref(), P(X), P(G), M, P(A), P(B), r, alpha, P(t), P(gx),
                                                  P(dA), P(dB), stream)
        else:
            wsb = lq.lib.lq_backward_workspace(qw.ref(), M, r)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            st = lq.lib.lq_qlora_backward(qw.ref(), P(X), P(G), M, P(A), P(B), r, alpha, P(t), P(gx), P(dA),
                                          P(dB), P(ws), wsb, stream)
        assert st == 0, st
        torch.cuda.synchronize()
        res.append([None if x is None else (x.view(torch.int16) if x.dtype == torch.bfloat16 else x).cpu().numpy()
                    for x in (gx, dA, dB)])
    return res


def assert_same(res):
    for a, b in zip(*res):
        assert (a is None) == (b is None)
        if a is not None:
            assert np.array_equal(a, b)


def test_noalloc_backward_equals_workspace_backward(lq, torch):
    # 1: the q_proj shape (4096 x 4096, 2048 tokens, r = 16), t saved
    W, X, G, A, B, t = layer_inputs(torch, 1, 4096, 4096, 2048, 16)
    qw = lq.QWeight.from_weight(W)
    assert_same(both(lq, torch, qw, X, G, A, B, t, 16, 32.0))
    # 2: smaller, ragged, t recomputed from X and A
    W, X, G, A, B, t = layer_inputs(torch, 2, 264, 320, 70, 24)
    qw = lq.QWeight.from_weight(W)
    assert_same(both(lq, torch, qw, X, G, A, B, None, 24, 8.0))
    # 3: smaller still, float32 block constants, dA only
    W, X, G, A, B, t = layer_inputs(torch, 3, 128, 192, 33, 16)
    qw = lq.QWeight.from_weight(W, double_quantize=False)
    assert_same(both(lq, torch, qw, X, G, A, B, t, 16, 32.0, need=(False, True, False)))


def test_noalloc_backward_codebook_weight(lq, torch):
    # the scratch also holds the dequantized copy of a codebook weight
    W, X, G, A, B, t = layer_inputs(torch, 4, 256, 384, 96, 16)
    rng = np.random.default_rng(4)
    bits = torch.from_numpy(rng.integers(1, 5, 256).astype(np.uint8)).cuda()
    levels, thresholds, _ = lq.lloyd_codebooks(W, bits)
    qw = lq.QWeight.from_codebook(W, bits, thresholds, levels)
    assert_same(both(lq, torch, qw, X, G, A, B, t, 16, 32.0))
    # and a second, smaller call after it
    W, X, G, A, B, t = layer_inputs(torch, 5, 64, 128, 17, 8)
    qw = lq.QWeight.from_weight(W)
    assert_same(both(lq, torch, qw, X, G, A, B, t, 8, 16.0))
