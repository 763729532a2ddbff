"""CPU tests of the C-ABI library: it loads, exports every entry point that
include/lq.h declares, its host tables equal the oracle's, its size queries
follow the closed forms, and argument validation rejects bad calls before
anything is launched (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lq.h")


@pytest.fixture(scope="module")
def lq():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "lq_build", os.path.join(ROOT, "quantized_lora_fine_lq_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    if not os.path.exists(build.LIB):
        build.build()
    import quantized_lora_fine_lq_amd as mod
    return mod


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s+(lq_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lq):
    names = declared_symbols()
    assert len(names) == 38
    dbg = lq.load_debug_library()
    for name in names:
        assert hasattr(lq.lib, name), name
        assert hasattr(dbg, name), name
        assert name in lq.SIGNATURES, name


def test_status_strings(lq):
    for s in (0, -1, -2, -3, -4, -5):
        assert lq.status_string(s) and lq.status_string(s) != "unknown status"
    assert lq.status_string(42) == "unknown status"
    assert lq.lib.lq_version() >= 100


def test_library_nf4_table_equals_oracle(lq):
    # the library builds its table with its own quantile routine (bisection on
    # erfc); the oracle uses scipy's ndtri. Both must round to the same float32.
    from oracle import nf4
    levels, thresholds = lq.nf4_table()
    assert np.array_equal(np.array(levels, dtype=np.float32), nf4.levels())
    assert np.array_equal(np.array(thresholds, dtype=np.float32), nf4.thresholds())


def test_sizes_closed_form(lq):
    s = lq.sizes(28672, 8192, 4)
    assert s["code_bytes"] == 117440512
    assert s["n_blocks"] == 3670016 and s["n_dq_blocks"] == 14336
    assert s["dq_const_bytes"] == 3670016 + 4 * 14336 + 4
    assert abs(s["const_bits_per_param_dq"] - 0.126953125) < 1e-15
    assert round(s["const_bits_per_param_dq"], 3) == 0.127
    assert s["const_bits_per_param_fp32"] == 0.5
    # LowRA-style mix: bits per weight from the code bytes
    s1 = lq.sizes(4096, 4096, 1)
    assert s1["code_bytes"] == 4096 * 4096 // 8


def test_validation_errors_without_launch(lq):
    L = lq.lib
    vp = ctypes.c_void_p
    fake = vp(0x1000)   # never dereferenced: every call below fails validation
    null = vp(None)
    assert L.lq_sizes(10, 64, 4, None) == lq.LQ_ERR_ARG
    assert L.lq_sizes(10, 65, 4, ctypes.byref(lq.lq_sizes_t())) == lq.LQ_ERR_SHAPE
    assert L.lq_quantize_nf4(null, 0, 4, 64, 64, fake, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_quantize_nf4(fake, 7, 4, 64, 64, fake, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_quantize_nf4(fake, 0, 4, 96, 64, fake, fake, null) == lq.LQ_ERR_SHAPE
    assert L.lq_quantize_nf4(fake, 0, 0, 64, 64, fake, fake, null) == lq.LQ_ERR_SHAPE
    assert L.lq_quantize_nf4(fake, 0, 4, 64, 32, fake, fake, null) == lq.LQ_ERR_UNSUPPORTED
    # AQLoRA profiling pass: 2 doubles per 64 blocks of workspace
    assert L.lq_profile_workspace(64, 4096, 64) == 2 * 64 * 8   # 4096 blocks = 64 workgroups
    assert L.lq_profile_workspace(4, 96, 64) == 0
    assert L.lq_profile_nf4(fake, 0, 4, 4096, 64, 0.01, fake, fake, 63, null) == lq.LQ_ERR_WORKSPACE
    assert L.lq_profile_nf4(fake, 0, 4, 4096, 32, 0.01, fake, fake, 64, null) == lq.LQ_ERR_UNSUPPORTED
    assert L.lq_profile_nf4(fake, 0, 4, 100, 64, 0.01, fake, fake, 64, null) == lq.LQ_ERR_SHAPE
    assert L.lq_profile_nf4(fake, 0, 4, 4096, 64, 0.01, null, fake, 64, null) == lq.LQ_ERR_ARG
    assert L.lq_profile_nf4(fake, 7, 4, 4096, 64, 0.01, fake, fake, 64, null) == lq.LQ_ERR_ARG
    assert L.lq_double_quant_workspace(1000, 256) >= 8 * 4
    assert L.lq_double_quant_workspace(1000, 128) == 0
    assert L.lq_double_quant(fake, 1000, 128, fake, fake, fake, fake, 1 << 20, null) == lq.LQ_ERR_UNSUPPORTED
    assert L.lq_double_quant(fake, 1000, 256, fake, fake, fake, fake, 8, null) == lq.LQ_ERR_WORKSPACE
    assert L.lq_double_quant(fake, 0, 256, fake, fake, fake, fake, 1 << 20, null) == lq.LQ_ERR_SHAPE
    assert L.lq_double_quant(null, 10, 256, fake, fake, fake, fake, 1 << 20, null) == lq.LQ_ERR_ARG
    dqd = L.lq_double_quant_dequant
    assert dqd(fake, 1000, 128, fake, fake, fake, fake, fake, fake, 1 << 20, null) == lq.LQ_ERR_UNSUPPORTED
    assert dqd(fake, 1000, 256, fake, fake, fake, fake, fake, fake, 8, null) == lq.LQ_ERR_WORKSPACE
    assert dqd(fake, 0, 256, fake, fake, fake, fake, fake, fake, 1 << 20, null) == lq.LQ_ERR_SHAPE
    assert dqd(fake, 10, 256, fake, fake, fake, null, fake, fake, 1 << 20, null) == lq.LQ_ERR_ARG
    assert dqd(fake, 10, 256, fake, fake, fake, fake, null, fake, 1 << 20, null) == lq.LQ_ERR_ARG

    def qw(**kw):
        d = dict(format=0, blocksize=64, N=128, K=256, codes=0x1000, absmax=0x1000, absmax_q=None,
                 dq_scale=None, dq_mean=None, dq_blocksize=256, reserved0=0, row_bits=None,
                 row_offset=None, levels=None)
        d.update(kw)
        return lq.lq_qweight(**d)

    assert L.lq_dequant(None, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_dequant(ctypes.byref(qw(format=5)), fake, null) == lq.LQ_ERR_ARG
    assert L.lq_dequant(ctypes.byref(qw(blocksize=128)), fake, null) == lq.LQ_ERR_UNSUPPORTED
    assert L.lq_dequant(ctypes.byref(qw(K=100)), fake, null) == lq.LQ_ERR_SHAPE
    assert L.lq_dequant(ctypes.byref(qw(absmax=None)), fake, null) == lq.LQ_ERR_ARG
    assert L.lq_dequant(ctypes.byref(qw(absmax=None, absmax_q=1, dq_scale=1, dq_mean=1, dq_blocksize=64)),
                        fake, null) == lq.LQ_ERR_UNSUPPORTED
    assert L.lq_dequant(ctypes.byref(qw(format=1)), fake, null) == lq.LQ_ERR_ARG
    assert L.lq_dequant(ctypes.byref(qw()), null, null) == lq.LQ_ERR_ARG

    w = qw()
    ws = L.lq_forward_workspace(ctypes.byref(w), 16, 16)
    assert ws >= 16 * 16 * 4
    assert L.lq_forward_workspace(ctypes.byref(w), 16, 0) == 0
    assert L.lq_forward_workspace(ctypes.byref(w), 16, 129) == 0
    args = (ctypes.byref(w), fake, 16, fake, fake, 16, 32.0, fake, 1, null, fake, ws, null)
    bad_r = list(args); bad_r[5] = 0
    assert L.lq_qlora_forward(*bad_r) == lq.LQ_ERR_SHAPE
    bad_h = list(args); bad_h[8] = 2
    assert L.lq_qlora_forward(*bad_h) == lq.LQ_ERR_UNSUPPORTED
    bad_ws = list(args); bad_ws[11] = ws - 1
    assert L.lq_qlora_forward(*bad_ws) == lq.LQ_ERR_WORKSPACE
    bad_x = list(args); bad_x[1] = null
    assert L.lq_qlora_forward(*bad_x) == lq.LQ_ERR_ARG
    bad_m = list(args); bad_m[2] = 0
    assert L.lq_qlora_forward(*bad_m) == lq.LQ_ERR_SHAPE

    wsb = L.lq_backward_workspace(ctypes.byref(w), 64, 16)
    assert wsb >= 2 * 64 * 16 * 4
    bargs = [ctypes.byref(w), fake, fake, 64, fake, fake, 16, 32.0, null, fake, fake, fake, fake, wsb, null]
    b1 = list(bargs); b1[1] = null      # X needed for dA and for recomputing t
    assert L.lq_qlora_backward(*b1) == lq.LQ_ERR_ARG
    b2 = list(bargs); b2[13] = 0
    assert L.lq_qlora_backward(*b2) == lq.LQ_ERR_WORKSPACE
    w_odd = qw(N=100)                   # backward needs N % 8 == 0
    b3 = list(bargs); b3[0] = ctypes.byref(w_odd)
    assert L.lq_qlora_backward(*b3) == lq.LQ_ERR_SHAPE
    # a codebook weight is dequantized into the workspace: N * K * 2 more bytes
    wc = qw(format=1, row_bits=1, row_offset=0x1000, levels=0x1000)
    wsc = L.lq_backward_workspace(ctypes.byref(wc), 64, 16)
    assert wsc == wsb + 128 * 256 * 2
    b4 = list(bargs); b4[0] = ctypes.byref(wc)
    assert L.lq_qlora_backward(*b4) == lq.LQ_ERR_WORKSPACE
    # split forward stages: NF4 needs no workspace (the GEMM forms its LoRA
    # operands itself); a codebook weight is dequantized into N * K * 2 bytes
    assert L.lq_dequant_gemm_workspace(ctypes.byref(wc), 300, 16) == 128 * 256 * 2
    assert L.lq_dequant_gemm_workspace(ctypes.byref(wc), 16, 16) == 0   # decode GEMV: no weight copy
    assert L.lq_dequant_gemm_t_workspace(ctypes.byref(wc), 300, 16) == 128 * 256 * 2
    assert L.lq_dequant_gemm_workspace(ctypes.byref(w), 300, 16) == 0
    assert L.lq_dequant_gemm_workspace(ctypes.byref(w), 16, 16) == 0
    assert L.lq_dequant_gemm_t_workspace(ctypes.byref(w), 300, 16) == 0
    assert L.lq_lora_down_workspace(300, 256, 16) == 0
    wg = L.lq_dequant_gemm_workspace(ctypes.byref(wc), 300, 16)
    gargs = [ctypes.byref(wc), fake, 300, fake, fake, 16, 32.0, fake, 1, fake, wg, null]
    g1 = list(gargs); g1[10] = wg - 1
    assert L.lq_dequant_gemm(*g1) == lq.LQ_ERR_WORKSPACE
    g2 = list(gargs); g2[9] = null
    assert L.lq_dequant_gemm(*g2) == lq.LQ_ERR_WORKSPACE
    g3 = list(gargs); g3[5] = 129
    assert L.lq_dequant_gemm(*g3) == lq.LQ_ERR_SHAPE
    wt = L.lq_dequant_gemm_t_workspace(ctypes.byref(wc), 300, 16)
    targs = [ctypes.byref(wc), fake, 300, fake, fake, 16, 32.0, fake, fake, wt, null]
    t1 = list(targs); t1[9] = wt - 1
    assert L.lq_dequant_gemm_t(*t1) == lq.LQ_ERR_WORKSPACE
    t2 = list(targs); t2[0] = ctypes.byref(w_odd)
    assert L.lq_dequant_gemm_t(*t2) == lq.LQ_ERR_SHAPE

    assert L.lq_quantize_codebook(fake, 0, 4, 64, 64, null, fake, fake, fake, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_quantize_codebook(fake, 0, 4, 60, 64, fake, fake, fake, fake, fake, null) == lq.LQ_ERR_SHAPE
    assert L.lq_quantize_codebook(fake, 0, 4, 64, 16, fake, fake, fake, fake, fake, null) == lq.LQ_ERR_UNSUPPORTED

    largs = [fake, 0, 4, 64, 64, fake, 100, fake, fake, null, null]   # iterations may be NULL
    for pos in (0, 5, 7, 8):
        a = list(largs); a[pos] = null
        assert L.lq_lloyd_codebooks(*a) == lq.LQ_ERR_ARG
    for it in (0, -1, 100001):
        a = list(largs); a[6] = it
        assert L.lq_lloyd_codebooks(*a) == lq.LQ_ERR_ARG
    a = list(largs); a[1] = 7
    assert L.lq_lloyd_codebooks(*a) == lq.LQ_ERR_ARG
    for n, k in ((0, 64), (4, 0), (4, 96), (1 << 31, 64)):
        a = list(largs); a[2] = n; a[3] = k
        assert L.lq_lloyd_codebooks(*a) == lq.LQ_ERR_SHAPE
    a = list(largs); a[4] = 32
    assert L.lq_lloyd_codebooks(*a) == lq.LQ_ERR_UNSUPPORTED
    a = list(largs); a[3] = 16384 + 64
    assert L.lq_lloyd_codebooks(*a) == lq.LQ_ERR_UNSUPPORTED


def test_lowrank_validation(lq):
    """Low-rank initialisation entry points: argument checks before any launch."""
    L = lq.lib
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(None)
    assert L.lq_lowrank_sub(null, 4, 64, fake, fake, 2, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_lowrank_sub(fake, 4, 64, null, fake, 2, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_lowrank_sub(fake, 4, 66, fake, fake, 2, fake, null) == lq.LQ_ERR_SHAPE
    assert L.lq_lowrank_sub(fake, 4, 64, fake, fake, 129, fake, null) == lq.LQ_ERR_SHAPE
    assert L.lq_residual(fake, null, 64, fake, null) == lq.LQ_ERR_ARG
    assert L.lq_residual(fake, fake, 62, fake, null) == lq.LQ_ERR_SHAPE

    # l even, r <= l <= min(N, K, 96)
    assert L.lq_svd_lowrank_workspace(256, 512, 16, 32) > 0
    for (N, K, r, l) in ((256, 512, 16, 15), (256, 512, 16, 33), (256, 512, 0, 32), (16, 512, 8, 32),
                         (256, 24, 8, 32)):
        assert L.lq_svd_lowrank_workspace(N, K, r, l) == 0
    ws = L.lq_svd_lowrank_workspace(256, 512, 16, 32)
    sargs = [fake, 256, 512, 16, 32, 8, fake, fake, fake, fake, fake, ws, null]
    s1 = list(sargs); s1[6] = null
    assert L.lq_svd_lowrank(*s1) == lq.LQ_ERR_ARG
    s2 = list(sargs); s2[4] = 98
    assert L.lq_svd_lowrank(*s2) == lq.LQ_ERR_UNSUPPORTED
    s3 = list(sargs); s3[4] = 8
    assert L.lq_svd_lowrank(*s3) == lq.LQ_ERR_SHAPE        # l < r
    s4 = list(sargs); s4[5] = -1
    assert L.lq_svd_lowrank(*s4) == lq.LQ_ERR_ARG
    s5 = list(sargs); s5[11] = ws - 1
    assert L.lq_svd_lowrank(*s5) == lq.LQ_ERR_WORKSPACE

    wl = L.lq_loftq_workspace(256, 512, 16, 32, 1)
    assert wl > ws + 256 * 512 * 6
    assert L.lq_loftq_workspace(256, 500, 16, 32, 1) == 0   # K % 64
    largs = [fake, 256, 512, 64, 1, 16, 32, 5, 8, fake, fake, fake, fake, fake, fake, fake, fake, fake, null,
             fake, wl, null]
    l1 = list(largs); l1[12] = null                         # double quant needs its outputs
    assert L.lq_loftq_init(*l1) == lq.LQ_ERR_ARG
    # without double quant the DQ outputs may be NULL (then only the workspace check is left)
    l2 = list(largs); l2[4] = 0; l2[12] = null; l2[13] = null; l2[14] = null; l2[20] = 1
    assert L.lq_loftq_init(*l2) == lq.LQ_ERR_WORKSPACE
    l3 = list(largs); l3[7] = 0
    assert L.lq_loftq_init(*l3) == lq.LQ_ERR_ARG
    l4 = list(largs); l4[3] = 32
    assert L.lq_loftq_init(*l4) == lq.LQ_ERR_UNSUPPORTED
    l5 = list(largs); l5[20] = wl - 1
    assert L.lq_loftq_init(*l5) == lq.LQ_ERR_WORKSPACE


def test_workspace_queries_deterministic(lq):
    w = lq.lq_qweight(0, 64, 4096, 4096, 0x1000, 0x1000, None, None, None, 256, 0, None, None, None)
    a = [lq.lib.lq_forward_workspace(ctypes.byref(w), 2048, 16) for _ in range(3)]
    b = [lq.lib.lq_backward_workspace(ctypes.byref(w), 2048, 16) for _ in range(3)]
    assert len(set(a)) == 1 and len(set(b)) == 1 and a[0] > 0 and b[0] > 0


def test_loraquant_validation(lq):
    L = lq.lib
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(None)
    assert L.lq_loraquant_workspace(256, 512, 16) > 0
    assert L.lq_loraquant_workspace(250, 512, 16) == 0     # N % 64
    assert L.lq_loraquant_workspace(256, 512, 65) == 0     # r > 64
    ws = L.lq_loraquant_workspace(256, 512, 16)
    args = [fake, fake, 256, 512, 16, 0.9, -1, 3, 1] + [fake] * 15 + [fake, ws, null]
    a = list(args); a[9] = null
    assert L.lq_loraquant(*a) == lq.LQ_ERR_ARG
    a = list(args); a[7] = 5
    assert L.lq_loraquant(*a) == lq.LQ_ERR_ARG
    a = list(args); a[6] = 17                              # h > r
    assert L.lq_loraquant(*a) == lq.LQ_ERR_ARG
    a = list(args); a[3] = 500
    assert L.lq_loraquant(*a) == lq.LQ_ERR_SHAPE
    a = list(args); a[4] = 65
    assert L.lq_loraquant(*a) == lq.LQ_ERR_UNSUPPORTED
    a = list(args); a[2] = 16448                           # beyond the codebook learner's row length
    assert L.lq_loraquant(*a) == lq.LQ_ERR_UNSUPPORTED
    assert L.lq_loraquant_workspace(16448, 512, 16) == 0
    a = list(args); a[25] = ws - 1
    assert L.lq_loraquant(*a) == lq.LQ_ERR_WORKSPACE
    dws = L.lq_loraquant_dequant_workspace(256, 512, 16)
    assert dws == 256 * 16 * 2
    dargs = [fake] * 9 + [256, 512, 16, fake, fake, fake, dws, null]
    d = list(dargs); d[12] = null
    assert L.lq_loraquant_dequant(*d) == lq.LQ_ERR_ARG
    d = list(dargs); d[8] = null
    assert L.lq_loraquant_dequant(*d) == lq.LQ_ERR_ARG
    d = list(dargs); d[15] = dws - 1
    assert L.lq_loraquant_dequant(*d) == lq.LQ_ERR_WORKSPACE


# ---- alignment, the host table check and the LQ_DEBUG build ----------------

def _libs(lq):
    return [("release", lq.lib), ("debug", lq.load_debug_library())]


def test_debug_build_flag(lq):
    assert lq.lib.lq_debug_build() == 0
    assert lq.load_debug_library().lq_debug_build() == 1
    v = ctypes.c_uint32(0)
    # the release build has no flag word; neither build accepts a null output
    assert lq.lib.lq_debug_flags(ctypes.byref(v), 0) == lq.LQ_ERR_UNSUPPORTED
    assert lq.load_debug_library().lq_debug_flags(None, 0) == lq.LQ_ERR_ARG


@pytest.mark.parametrize("which", ["release", "debug"])
def test_misaligned_pointers_rejected_before_launch(lq, which):
    L = dict(_libs(lq))[which]
    vp = ctypes.c_void_p
    a = 0x10000            # 16-byte aligned fake device address (never dereferenced)
    null = vp(None)
    ARG = lq.LQ_ERR_ARG
    # quantizer: float32 W needs 16 bytes, bf16 W 8, the codes 8
    assert L.lq_quantize_nf4(vp(a + 8), 0, 4, 64, 64, vp(a), vp(a), null) == ARG
    assert L.lq_quantize_nf4(vp(a + 4), 1, 4, 64, 64, vp(a), vp(a), null) == ARG
    assert L.lq_quantize_nf4(vp(a), 0, 4, 64, 64, vp(a + 4), vp(a), null) == ARG
    assert L.lq_quantize_nf4(vp(a), 0, 4, 64, 64, vp(a), vp(a + 2), null) == ARG
    assert L.lq_profile_nf4(vp(a + 4), 0, 4, 4096, 64, 0.01, vp(a), vp(a), 1 << 20, null) == ARG
    assert L.lq_double_quant(vp(a + 2), 1000, 256, vp(a), vp(a), vp(a), vp(a), 1 << 20, null) == ARG
    # double quant + dequant: the codes and the bf16 output need 16 bytes
    for i in (0, 6, 7):
        args = [vp(a), 1000, 256, vp(a), vp(a), vp(a), vp(a), vp(a), vp(a), 1 << 20, null]
        args[i] = vp(a + (2 if i == 0 else 8))
        assert L.lq_double_quant_dequant(*args) == ARG

    def qw(**kw):
        d = dict(format=0, blocksize=64, N=128, K=256, codes=a, absmax=a, absmax_q=None,
                 dq_scale=None, dq_mean=None, dq_blocksize=256, reserved0=0, row_bits=None,
                 row_offset=None, levels=None)
        d.update(kw)
        return lq.lq_qweight(**d)

    assert L.lq_dequant(ctypes.byref(qw(codes=a + 4)), vp(a), null) == ARG
    assert L.lq_dequant(ctypes.byref(qw(absmax=a + 2)), vp(a), null) == ARG
    assert L.lq_dequant(ctypes.byref(qw(absmax=None, absmax_q=a + 1, dq_scale=a, dq_mean=a)), vp(a), null) == ARG
    assert L.lq_dequant(ctypes.byref(qw()), vp(a + 8), null) == ARG
    w = qw()
    ws = L.lq_forward_workspace(ctypes.byref(w), 16, 16)
    good = dict(X=a, A=a, B=a, H=a, t=a, ws=a)
    for bad in ("X", "A", "B", "H", "t", "ws"):
        p = dict(good)
        p[bad] = a + 2
        assert L.lq_qlora_forward(ctypes.byref(w), vp(p["X"]), 16, vp(p["A"]), vp(p["B"]), 16, 32.0, vp(p["H"]), 1,
                                  vp(p["t"]), vp(p["ws"]), ws, null) == ARG, bad
        if bad != "A":
            assert L.lq_dequant_gemm(ctypes.byref(w), vp(p["X"]), 16, vp(p["t"]), vp(p["B"]), 16, 32.0, vp(p["H"]),
                                     1, vp(p["ws"]), 1 << 20, null) == ARG, bad
    # a float32 H needs only 4 bytes: that call gets past the alignment checks
    # and stops at the next one (a workspace one byte short); nothing launches
    st = L.lq_qlora_forward(ctypes.byref(w), vp(a), 16, vp(a), vp(a), 16, 32.0, vp(a + 4), 0, null, vp(a), ws - 1,
                            null)
    assert st == lq.LQ_ERR_WORKSPACE
    bws = L.lq_backward_workspace(ctypes.byref(w), 64, 16)
    for bad in range(9):
        p = [a] * 9
        p[bad] += 2
        X, G, A, B, t, gx, dA, dB, wsp = p
        assert L.lq_qlora_backward(ctypes.byref(w), vp(X), vp(G), 64, vp(A), vp(B), 16, 32.0, vp(t), vp(gx),
                                   vp(dA), vp(dB), vp(wsp), bws, null) == ARG, bad
    assert L.lq_dequant_gemm_t(ctypes.byref(w), vp(a + 8), 64, vp(a), vp(a), 16, 32.0, vp(a), vp(a), 0, null) == ARG
    assert L.lq_lora_down(vp(a), 16, 256, vp(a + 8), 16, vp(a), null, 0, null) == ARG
    # the codebook quantizer takes W at any element alignment (this call stops
    # at the blocksize check, after the alignment checks), codes at 4 bytes
    assert L.lq_quantize_codebook(vp(a + 4), 0, 4, 64, 32, vp(a), vp(a), vp(a), vp(a), vp(a), null) == \
        lq.LQ_ERR_UNSUPPORTED
    assert L.lq_quantize_codebook(vp(a + 2), 0, 4, 64, 64, vp(a), vp(a), vp(a), vp(a), vp(a), null) == ARG
    assert L.lq_quantize_codebook(vp(a), 0, 4, 64, 64, vp(a), vp(a + 4), vp(a), vp(a), vp(a), null) == ARG
    assert L.lq_quantize_codebook(vp(a), 0, 4, 64, 64, vp(a), vp(a), vp(a), vp(a + 2), vp(a), null) == ARG
    assert L.lq_lowrank_sub(vp(a + 4), 4, 64, vp(a), vp(a), 2, vp(a), null) == ARG
    assert L.lq_residual(vp(a), vp(a + 4), 64, vp(a), null) == ARG


def test_host_codebook_table_check(lq):
    L = lq.lib
    N, K = 4, 128
    bits = np.array([1, 4, 3, 2], dtype=np.uint8)
    off = np.concatenate([[0], np.cumsum(K * bits.astype(np.int64) // 8)]).astype(np.int64)
    T = np.full((N, 15), 3.0, dtype=np.float32)
    for i, b in enumerate(bits):
        T[i, :(1 << b) - 1] = np.linspace(-0.9, 0.9, (1 << b) - 1)
    P = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    assert L.lq_check_codebook_tables(N, K, P(bits), P(off), P(T)) == lq.LQ_OK
    assert L.lq_check_codebook_tables(N, K, P(bits), P(off), None) == lq.LQ_OK
    assert L.lq_check_codebook_tables(N, 100, P(bits), P(off), None) == lq.LQ_ERR_SHAPE
    assert L.lq_check_codebook_tables(N, K, None, P(off), None) == lq.LQ_ERR_ARG
    b2 = bits.copy(); b2[2] = 5
    assert L.lq_check_codebook_tables(N, K, P(b2), P(off), None) == lq.LQ_ERR_ARG
    b2[2] = 0
    assert L.lq_check_codebook_tables(N, K, P(b2), P(off), None) == lq.LQ_ERR_ARG
    o2 = off.copy(); o2[2] += 8
    assert L.lq_check_codebook_tables(N, K, P(bits), P(o2), None) == lq.LQ_ERR_ARG
    o2 = off.copy(); o2[0] = 8; o2[1:] += 8
    assert L.lq_check_codebook_tables(N, K, P(bits), P(o2), None) == lq.LQ_ERR_ARG
    T2 = T.copy(); T2[1, 5] = T2[1, 4]          # a tie is not strictly increasing
    assert L.lq_check_codebook_tables(N, K, P(bits), P(off), P(T2)) == lq.LQ_ERR_ARG
    T2 = T.copy(); T2[2, 3] = np.nan
    assert L.lq_check_codebook_tables(N, K, P(bits), P(off), P(T2)) == lq.LQ_ERR_ARG
    T2 = T.copy(); T2[0, 1:] = -5.0             # unused slots of a 1-bit row are not checked
    assert L.lq_check_codebook_tables(N, K, P(bits), P(off), P(T2)) == lq.LQ_OK


def test_noalloc_backward_refuses_shapes_beyond_its_scratch(lq):
    """The no-allocation backward checks its workspace need against the
    library's fixed scratch before touching the device (fake pointers: no
    call below gets past validation)."""
    L = lq.lib
    vp = ctypes.c_void_p
    a = vp(0x10000)
    null = vp(None)

    def qw(N, K, fmt=0):
        return lq.lq_qweight(format=fmt, blocksize=64, N=N, K=K, codes=0x10000, absmax=None, absmax_q=0x10000,
                             dq_scale=0x10000, dq_mean=0x10000, dq_blocksize=256, reserved0=0,
                             row_bits=0x10000 if fmt else None, row_offset=0x10000 if fmt else None,
                             levels=0x10000 if fmt else None)
    limit = lq.LQ_NOALLOC_SCRATCH_BYTES
    fits = [(4096, 4096, 2048, 16), (11008, 4096, 4096, 64), (4096, 11008, 4096, 64)]
    for N, K, M, r in fits:
        w = qw(N, K)
        need = L.lq_qlora_backward_noalloc_bytes(ctypes.byref(w), M, r)
        assert need == L.lq_backward_workspace(ctypes.byref(w), M, r)
        assert 0 < need <= limit
    big = qw(16384, 16384)
    assert L.lq_qlora_backward_noalloc_bytes(ctypes.byref(big), 8192, 128) > limit
    assert L.lq_qlora_backward_noalloc(ctypes.byref(big), a, a, 8192, a, a, 128, 16.0, a, a, a, a, null) == \
        lq.LQ_ERR_WORKSPACE
    # the codebook format also holds the dequantized weight (N K 2 bytes)
    cb = qw(11008, 4096, fmt=1)
    assert L.lq_qlora_backward_noalloc(ctypes.byref(cb), a, a, 4096, a, a, 64, 16.0, a, a, a, a, null) == \
        lq.LQ_ERR_WORKSPACE
    # argument errors come first, as in lq_qlora_backward
    assert L.lq_qlora_backward_noalloc(None, a, a, 64, a, a, 16, 32.0, a, a, a, a, null) == lq.LQ_ERR_ARG
    assert L.lq_qlora_backward_noalloc(ctypes.byref(big), a, vp(0x10002), 64, a, a, 16, 32.0, a, a, a, a, null) == \
        lq.LQ_ERR_ARG
    assert L.lq_qlora_backward_noalloc(ctypes.byref(big), a, a, 64, a, a, 0, 32.0, a, a, a, a, null) == \
        lq.LQ_ERR_SHAPE


def test_codebook_forward_workspace_by_path(lq, monkeypatch):
    """A codebook weight at decode sizes (M <= 16) goes through the GEMV,
    which needs no bfloat16 copy of the weight; larger M (or the GEMM
    forced) sizes the workspace for the dequantized weight."""
    monkeypatch.delenv("LQ_FORCE_PATH", raising=False)
    N, K = 512, 1024
    w = lq.lq_qweight(1, 64, N, K, 0x1000, 0x1000, None, None, None, 256, 0, 0x1000, 0x1000, 0x1000)
    small = lq.lib.lq_forward_workspace(ctypes.byref(w), 16, 16)
    assert 16 * 16 * 4 <= small < N * K * 2
    assert lq.lib.lq_dequant_gemm_workspace(ctypes.byref(w), 16, 16) == 0
    assert lq.lib.lq_forward_workspace(ctypes.byref(w), 17, 16) >= N * K * 2
    monkeypatch.setenv("LQ_FORCE_PATH", "gemm")
    assert lq.lib.lq_forward_workspace(ctypes.byref(w), 16, 16) >= N * K * 2
    # K past the GEMV's LDS budget: the GEMM path at every M
    monkeypatch.delenv("LQ_FORCE_PATH")
    wide = lq.lq_qweight(1, 64, 16, 32768, 0x1000, 0x1000, None, None, None, 256, 0, 0x1000, 0x1000, 0x1000)
    assert lq.lib.lq_forward_workspace(ctypes.byref(wide), 1, 16) >= 16 * 32768 * 2


def test_split_schedule_workspace(lq, monkeypatch):
    """The GEMM's schedule on 8 XCDs of 32 CUs: when an XCD's last round of
    256 x 128 tiles would be at most half full, its last tiles run as two
    halves of the contraction, whose float32 partial sums (2 x 256 x 128 per
    split tile) live in the workspace. q_proj (256 tiles, 32 per XCD) splits
    none; mlp_up forward and mlp_down's grad_X (1376 tiles, 172 per XCD:
    5 rounds and 12) split 12 per XCD; 1376 tiles with K = 960 (15 steps)
    split none."""
    monkeypatch.delenv("LQ_FORCE_PATH", raising=False)
    L = lq.lib

    def nf4(N, K):
        return lq.lq_qweight(0, 64, N, K, 0x1000, None, 0x1000, 0x1000, 0x1000, 256, 0, None, None, None)
    part = 96 * 2 * 256 * 128 * 4
    assert L.lq_dequant_gemm_workspace(ctypes.byref(nf4(4096, 4096)), 2048, 16) == 0
    assert L.lq_dequant_gemm_workspace(ctypes.byref(nf4(11008, 4096)), 4096, 64) == part
    assert L.lq_dequant_gemm_workspace(ctypes.byref(nf4(11008, 960)), 4096, 64) == 0
    assert L.lq_dequant_gemm_t_workspace(ctypes.byref(nf4(4096, 11008)), 4096, 64) == part
    assert L.lq_dequant_gemm_t_workspace(ctypes.byref(nf4(11008, 4096)), 4096, 64) == 0
    # 264 tiles (33 per XCD): one split tile per XCD
    assert L.lq_dequant_gemm_workspace(ctypes.byref(nf4(132 * 128, 1024)), 512, 16) == 8 * 2 * 256 * 128 * 4
    # the backward's workspace carries the same partial sums for grad_X
    assert L.lq_backward_workspace(ctypes.byref(nf4(4096, 11008)), 4096, 64) > part
