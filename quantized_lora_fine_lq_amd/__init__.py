"""Python binding of liblq.so, the gfx950 quantized-LoRA hot path (include/lq.h).

Two layers, both argument marshalling only:

* ``lib`` -- the ctypes handle; ``lib.lq_quantize_nf4(...)`` etc. take raw
  device pointers exactly as declared in include/lq.h;
* tensor helpers (``quantize_nf4``, ``double_quant``, ``QWeight``,
  ``dequant``, ``qlora_forward``, ``qlora_backward``, ``quantize_codebook``)
  that allocate outputs and workspaces with PyTorch (device memory and the
  current stream are the only things taken from PyTorch) and call the same
  entry points. All arithmetic runs in the library's HIP kernels.

Importing fails loudly if liblq.so has not been built
(``python quantized_lora_fine_lq_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "liblq.so")
DEBUG_LIB_PATH = os.path.join(HERE, "lib", "liblq_debug.so")
LQ_DBG_NONFINITE, LQ_DBG_THRESHOLDS, LQ_DBG_ROW_BITS = 1, 2, 4
LQ_NOALLOC_SCRATCH_BYTES = 96 << 20

LQ_OK, LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH = 0, -1, -2, -3, -4, -5
LQ_F32, LQ_BF16, LQ_F16 = 0, 1, 2
LQ_FMT_NF4, LQ_FMT_CODEBOOK = 0, 1

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class lq_qweight(ctypes.Structure):
    _fields_ = [
        ("format", c_i32), ("blocksize", c_i32), ("N", c_i64), ("K", c_i64),
        ("codes", c_vp), ("absmax", c_vp), ("absmax_q", c_vp), ("dq_scale", c_vp),
        ("dq_mean", c_vp), ("dq_blocksize", c_i32), ("reserved0", c_i32),
        ("row_bits", c_vp), ("row_offset", c_vp), ("levels", c_vp),
    ]


class lq_sizes_t(ctypes.Structure):
    _fields_ = [
        ("n", c_i64), ("n_blocks", c_i64), ("n_dq_blocks", c_i64), ("code_bytes", c_i64),
        ("dq_const_bytes", c_i64), ("fp32_const_bytes", c_i64),
        ("const_bits_per_param_dq", ctypes.c_double), ("const_bits_per_param_fp32", ctypes.c_double),
    ]


QW_P = ctypes.POINTER(lq_qweight)

# name -> (restype, argtypes); the full export list of include/lq.h
SIGNATURES = {
    "lq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lq_version": (ctypes.c_int, []),
    "lq_nf4_table": (ctypes.c_int, [c_vp, c_vp]),
    "lq_sizes": (ctypes.c_int, [c_i64, c_i64, c_i32, ctypes.POINTER(lq_sizes_t)]),
    "lq_quantize_nf4": (ctypes.c_int, [c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp]),
    "lq_profile_workspace": (c_sz, [c_i64, c_i64, c_i32]),
    "lq_profile_nf4": (ctypes.c_int, [c_vp, c_i32, c_i64, c_i64, c_i32, ctypes.c_double, c_vp, c_vp, c_sz, c_vp]),
    "lq_double_quant_workspace": (c_sz, [c_i64, c_i32]),
    "lq_double_quant": (ctypes.c_int, [c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lq_double_quant_dequant": (ctypes.c_int, [c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                               c_vp]),
    "lq_dequant": (ctypes.c_int, [QW_P, c_vp, c_vp]),
    "lq_forward_workspace": (c_sz, [QW_P, c_i64, c_i32]),
    "lq_qlora_forward": (ctypes.c_int, [QW_P, c_vp, c_i64, c_vp, c_vp, c_i32, c_f32, c_vp, c_i32,
                                        c_vp, c_vp, c_sz, c_vp]),
    "lq_backward_workspace": (c_sz, [QW_P, c_i64, c_i32]),
    "lq_qlora_backward": (ctypes.c_int, [QW_P, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_f32, c_vp,
                                         c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lq_quantize_codebook": (ctypes.c_int, [c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp,
                                            c_vp, c_vp, c_vp]),
    "lq_lloyd_codebooks": (ctypes.c_int, [c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_i32, c_vp, c_vp,
                                          c_vp, c_vp]),
    "lq_lowrank_sub": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_i32, c_vp, c_vp]),
    "lq_residual": (ctypes.c_int, [c_vp, c_vp, c_i64, c_vp, c_vp]),
    "lq_svd_lowrank_workspace": (c_sz, [c_i64, c_i64, c_i32, c_i32]),
    "lq_svd_lowrank": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_sz, c_vp]),
    "lq_loftq_workspace": (c_sz, [c_i64, c_i64, c_i32, c_i32, c_i32]),
    "lq_loftq_init": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                     c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lq_loraquant_workspace": (c_sz, [c_i64, c_i64, c_i32]),
    "lq_loraquant": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i32, ctypes.c_double, c_i32, c_i32, c_i32,
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lq_loraquant_dequant_workspace": (c_sz, [c_i64, c_i64, c_i32]),
    "lq_loraquant_dequant": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                            c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "lq_lora_down_workspace": (c_sz, [c_i64, c_i64, c_i32]),
    "lq_lora_down": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "lq_dequant_gemm_workspace": (c_sz, [QW_P, c_i64, c_i32]),
    "lq_dequant_gemm": (ctypes.c_int, [QW_P, c_vp, c_i64, c_vp, c_vp, c_i32, c_f32, c_vp, c_i32,
                                       c_vp, c_sz, c_vp]),
    "lq_dequant_gemm_t_workspace": (c_sz, [QW_P, c_i64, c_i32]),
    "lq_dequant_gemm_t": (ctypes.c_int, [QW_P, c_vp, c_i64, c_vp, c_vp, c_i32, c_f32, c_vp,
                                         c_vp, c_sz, c_vp]),
    "lq_qlora_backward_noalloc_bytes": (c_sz, [QW_P, c_i64, c_i32]),
    "lq_qlora_backward_noalloc": (ctypes.c_int, [QW_P, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_f32, c_vp,
                                                 c_vp, c_vp, c_vp, c_vp]),
    "lq_check_codebook_tables": (ctypes.c_int, [c_i64, c_i64, c_vp, c_vp, c_vp]),
    "lq_debug_build": (ctypes.c_int, []),
    "lq_debug_flags": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]),
}


class LqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status} ({status_string(status)})")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python quantized_lora_fine_lq_amd/build.py`")
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


def load_debug_library() -> ctypes.CDLL:
    """The LQ_DEBUG build (same entry points and signatures as ``lib``)."""
    return _load(DEBUG_LIB_PATH)


def status_string(status: int) -> str:
    return lib.lq_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != LQ_OK:
        raise LqError(status, where)


def nf4_table():
    """(levels[16], thresholds[15]) as Python float lists (host call)."""
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(lib.lq_nf4_table(ctypes.cast(lv, c_vp), ctypes.cast(th, c_vp)), "lq_nf4_table")
    return list(lv), list(th)


def sizes(N: int, K: int, bits: int = 4) -> dict:
    out = lq_sizes_t()
    _check(lib.lq_sizes(N, K, bits, ctypes.byref(out)), "lq_sizes")
    return {f: getattr(out, f) for f, _ in lq_sizes_t._fields_}


# ---------------------------------------------------------------------------
# tensor helpers (PyTorch provides memory and the stream only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(dev=None):
    torch = _torch()
    return c_vp(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t) -> c_vp:
    return c_vp(t.data_ptr()) if t is not None else c_vp(None)


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: LQ_F32, torch.bfloat16: LQ_BF16, torch.float16: LQ_F16}[t.dtype]


def _contig_cuda(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t


def quantize_nf4(W, blocksize: int = 64):
    """W [N, K] (f32/bf16/f16) -> (codes uint8 [N*K/2], absmax f32 [N*K/64])."""
    torch = _torch()
    _contig_cuda(W, "W")
    N, K = W.shape
    codes = torch.empty(N * K // 2, dtype=torch.uint8, device=W.device)
    absmax = torch.empty(max(N * K // blocksize, 1), dtype=torch.float32, device=W.device)
    _check(lib.lq_quantize_nf4(_ptr(W), _dtype_code(W), N, K, blocksize, _ptr(codes), _ptr(absmax),
                               _stream(W.device)), "lq_quantize_nf4")
    return codes, absmax


def profile_nf4(W, tau: float = 0.01, blocksize: int = 64):
    """AQLoRA profiling pass of one layer: device float64 tensor
    [eps, fraction of |w| < tau]."""
    torch = _torch()
    _contig_cuda(W, "W")
    N, K = W.shape
    stats = torch.empty(2, dtype=torch.float64, device=W.device)
    ws_bytes = lib.lq_profile_workspace(N, K, blocksize)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=W.device)
    _check(lib.lq_profile_nf4(_ptr(W), _dtype_code(W), N, K, blocksize, float(tau), _ptr(stats), _ptr(ws),
                              ws_bytes, _stream(W.device)), "lq_profile_nf4")
    return stats


def double_quant(absmax, dq_blocksize: int = 256):
    """absmax f32 [n_b] -> (absmax_q uint8 [n_b], dq_scale f32 [n_d], dq_mean f32 [1])."""
    torch = _torch()
    _contig_cuda(absmax, "absmax")
    n_b = absmax.numel()
    n_d = (n_b + dq_blocksize - 1) // dq_blocksize
    q = torch.empty(n_b, dtype=torch.uint8, device=absmax.device)
    s2 = torch.empty(n_d, dtype=torch.float32, device=absmax.device)
    mu = torch.empty(1, dtype=torch.float32, device=absmax.device)
    ws_bytes = lib.lq_double_quant_workspace(n_b, dq_blocksize)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=absmax.device)
    _check(lib.lq_double_quant(_ptr(absmax), n_b, dq_blocksize, _ptr(q), _ptr(s2), _ptr(mu), _ptr(ws),
                               ws_bytes, _stream(absmax.device)), "lq_double_quant")
    return q, s2, mu


def double_quant_dequant(codes, absmax, shape, dq_blocksize: int = 256):
    """NF4 codes uint8 [n_b*32] and absmax f32 [n_b] -> (absmax_q, dq_scale, dq_mean, W' bf16 of `shape`):
    double quantization, then the dequantized weight from the new constants."""
    torch = _torch()
    _contig_cuda(absmax, "absmax")
    _contig_cuda(codes, "codes")
    n_b = absmax.numel()
    if codes.numel() != 32 * n_b or shape[0] * shape[1] != 64 * n_b:
        raise ValueError("codes, absmax and shape disagree")
    n_d = (n_b + dq_blocksize - 1) // dq_blocksize
    dev = absmax.device
    q = torch.empty(n_b, dtype=torch.uint8, device=dev)
    s2 = torch.empty(n_d, dtype=torch.float32, device=dev)
    mu = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=dev)
    ws_bytes = lib.lq_double_quant_workspace(n_b, dq_blocksize)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.lq_double_quant_dequant(_ptr(absmax), n_b, dq_blocksize, _ptr(q), _ptr(s2), _ptr(mu), _ptr(codes),
                                       _ptr(out), _ptr(ws), ws_bytes, _stream(dev)), "lq_double_quant_dequant")
    return q, s2, mu, out


class QWeight:
    """A quantized frozen weight: device tensors plus the lq_qweight view."""

    def __init__(self, N: int, K: int, codes, absmax=None, absmax_q=None, dq_scale=None,
                 dq_mean=None, fmt: int = LQ_FMT_NF4, row_bits=None, row_offset=None, levels=None):
        self.N, self.K, self.fmt = N, K, fmt
        self.codes, self.absmax = codes, absmax
        self.absmax_q, self.dq_scale, self.dq_mean = absmax_q, dq_scale, dq_mean
        self.row_bits, self.row_offset, self.levels = row_bits, row_offset, levels
        self.desc = lq_qweight(fmt, 64, N, K, _ptr(codes), _ptr(absmax), _ptr(absmax_q), _ptr(dq_scale),
                               _ptr(dq_mean), 256, 0, _ptr(row_bits), _ptr(row_offset), _ptr(levels))

    @property
    def device(self):
        return self.codes.device

    def ref(self):
        return ctypes.byref(self.desc)

    @classmethod
    def from_weight(cls, W, double_quantize: bool = True) -> "QWeight":
        """Quantize W [N, K] to NF4 (+ double quantization of the constants)."""
        N, K = W.shape
        codes, absmax = quantize_nf4(W)
        if not double_quantize:
            return cls(N, K, codes, absmax=absmax)
        q, s2, mu = double_quant(absmax)
        return cls(N, K, codes, absmax_q=q, dq_scale=s2, dq_mean=mu)

    @classmethod
    def from_codebook(cls, W, row_bits, thresholds, levels, double_quantize: bool = True) -> "QWeight":
        N, K = W.shape
        codes, absmax, row_offset = quantize_codebook(W, row_bits, thresholds)
        if not double_quantize:
            return cls(N, K, codes, absmax=absmax, fmt=LQ_FMT_CODEBOOK, row_bits=row_bits,
                       row_offset=row_offset, levels=levels)
        q, s2, mu = double_quant(absmax)
        return cls(N, K, codes, absmax_q=q, dq_scale=s2, dq_mean=mu, fmt=LQ_FMT_CODEBOOK,
                   row_bits=row_bits, row_offset=row_offset, levels=levels)


def dequant(qw: QWeight):
    torch = _torch()
    out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=qw.device)
    _check(lib.lq_dequant(qw.ref(), _ptr(out), _stream(qw.device)), "lq_dequant")
    return out


def qlora_forward(qw: QWeight, X, A, B, alpha: float, out_dtype=None, save_t: bool = True):
    """H = X W'^T + (alpha/r) (X A^T) B^T. Returns (H [M, N], t [M, r] f32 or None)."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    for n, t in (("X", X), ("A", A), ("B", B)):
        _contig_cuda(t, n)
    M, r = X.shape[0], A.shape[0]
    H = torch.empty(M, qw.N, dtype=out_dtype, device=X.device)
    t = torch.empty(M, r, dtype=torch.float32, device=X.device) if save_t else None
    ws_bytes = lib.lq_forward_workspace(qw.ref(), M, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=X.device)
    h_code = LQ_F32 if out_dtype == torch.float32 else LQ_BF16
    _check(lib.lq_qlora_forward(qw.ref(), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(H), h_code,
                                _ptr(t), _ptr(ws), ws_bytes, _stream(X.device)), "lq_qlora_forward")
    return H, t


def qlora_backward(qw: QWeight, X, G, A, B, alpha: float, t=None,
                   need_grad_x: bool = True, need_dA: bool = True, need_dB: bool = True):
    """Returns (grad_X bf16 [M, K] | None, dA f32 [r, K] | None, dB f32 [N, r] | None)."""
    torch = _torch()
    M, r = G.shape[0], A.shape[0]
    dev = G.device
    gx = torch.empty(M, qw.K, dtype=torch.bfloat16, device=dev) if need_grad_x else None
    dA = torch.empty(r, qw.K, dtype=torch.float32, device=dev) if need_dA else None
    dB = torch.empty(qw.N, r, dtype=torch.float32, device=dev) if need_dB else None
    ws_bytes = lib.lq_backward_workspace(qw.ref(), M, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.lq_qlora_backward(qw.ref(), _ptr(X), _ptr(G), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(t),
                                 _ptr(gx), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes, _stream(dev)),
           "lq_qlora_backward")
    return gx, dA, dB


def lora_down(X, A, t=None):
    """t = X A^T (float32 [M, r])."""
    torch = _torch()
    M, K = X.shape
    r = A.shape[0]
    t = torch.empty(M, r, dtype=torch.float32, device=X.device) if t is None else t
    ws_bytes = lib.lq_lora_down_workspace(M, K, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=X.device)
    _check(lib.lq_lora_down(_ptr(X), M, K, _ptr(A), r, _ptr(t), _ptr(ws), ws_bytes, _stream(X.device)),
           "lq_lora_down")
    return t


def dequant_gemm(qw: QWeight, X, t, B, alpha: float, out=None, out_dtype=None):
    """H = X W'^T + (alpha/r) t B^T given t."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, r = X.shape[0], t.shape[1]
    H = torch.empty(M, qw.N, dtype=out_dtype, device=X.device) if out is None else out
    h_code = LQ_F32 if H.dtype == torch.float32 else LQ_BF16
    ws_bytes = lib.lq_dequant_gemm_workspace(qw.ref(), M, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=X.device)
    _check(lib.lq_dequant_gemm(qw.ref(), _ptr(X), M, _ptr(t), _ptr(B), r, float(alpha), _ptr(H), h_code,
                               _ptr(ws), ws_bytes, _stream(X.device)), "lq_dequant_gemm")
    return H


def dequant_gemm_t(qw: QWeight, G, u, A, alpha: float, out=None):
    """grad_X = G W' + (alpha/r) u A given u = G B (bfloat16 [M, K])."""
    torch = _torch()
    M, r = G.shape[0], u.shape[1]
    gx = torch.empty(M, qw.K, dtype=torch.bfloat16, device=G.device) if out is None else out
    ws_bytes = lib.lq_dequant_gemm_t_workspace(qw.ref(), M, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=G.device)
    _check(lib.lq_dequant_gemm_t(qw.ref(), _ptr(G), M, _ptr(u), _ptr(A), r, float(alpha), _ptr(gx),
                                 _ptr(ws), ws_bytes, _stream(G.device)), "lq_dequant_gemm_t")
    return gx


def row_offsets(row_bits_host, K: int):
    """Byte offsets of each row's bit-planes (prefix sums of K*b/8), host list."""
    off = [0]
    for b in row_bits_host:
        off.append(off[-1] + K * int(b) // 8)
    return off


def lloyd_codebooks(W, row_bits, max_iters: int = 100, blocksize: int = 64):
    """Per-row weighted Lloyd-Max codebooks for W [N, K] (device) with
    row_bits uint8 [N] (device) -> (levels f32 [N, 16], thresholds f32 [N, 15],
    iterations int32 [N]), ready for quantize_codebook / QWeight.from_codebook."""
    torch = _torch()
    N, K = W.shape
    levels = torch.empty(N, 16, dtype=torch.float32, device=W.device)
    thresholds = torch.empty(N, 15, dtype=torch.float32, device=W.device)
    iters = torch.empty(N, dtype=torch.int32, device=W.device)
    _check(lib.lq_lloyd_codebooks(_ptr(W), _dtype_code(W), N, K, blocksize, _ptr(row_bits), int(max_iters),
                                  _ptr(levels), _ptr(thresholds), _ptr(iters), _stream(W.device)),
           "lq_lloyd_codebooks")
    return levels, thresholds, iters


def lowrank_sub(W, B, A):
    """float32(W - B A) with the rank-r product summed in float64."""
    torch = _torch()
    N, K = W.shape
    r = B.shape[1]
    out = torch.empty_like(W)
    _check(lib.lq_lowrank_sub(_ptr(W), N, K, _ptr(B) if r else None, _ptr(A) if r else None, r, _ptr(out),
                              _stream(W.device)), "lq_lowrank_sub")
    return out


def residual(W, Wd):
    """R = W - W' for a float32 W and a bfloat16 W'."""
    torch = _torch()
    R = torch.empty_like(W)
    _check(lib.lq_residual(_ptr(W), _ptr(Wd), W.numel(), _ptr(R), _stream(W.device)), "lq_residual")
    return R


def svd_lowrank(R, r: int, omega, power_iters: int = 8):
    """Rank-r SVD of R [N, K] (float32) by randomized subspace iteration from
    omega [K, l] -> (B [N, r], A [r, K], sigma [r]) with B A ~ the truncated SVD."""
    torch = _torch()
    N, K = R.shape
    l = omega.shape[1]
    B = torch.empty(N, r, dtype=torch.float32, device=R.device)
    A = torch.empty(r, K, dtype=torch.float32, device=R.device)
    sigma = torch.empty(r, dtype=torch.float32, device=R.device)
    ws_bytes = lib.lq_svd_lowrank_workspace(N, K, r, l)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=R.device)
    _check(lib.lq_svd_lowrank(_ptr(R), N, K, r, l, int(power_iters), _ptr(omega), _ptr(B), _ptr(A), _ptr(sigma),
                              _ptr(ws), ws_bytes, _stream(R.device)), "lq_svd_lowrank")
    return B, A, sigma


def loftq_init(W, r: int, omega, steps: int = 5, power_iters: int = 8, double_quant: bool = True,
               blocksize: int = 64):
    """LoftQ-style initialisation of W [N, K] (float32): returns (QWeight,
    B [N, r] f32, A [r, K] f32, sigma [r], objectives [steps] f64)."""
    torch = _torch()
    N, K = W.shape
    l = omega.shape[1]
    dev = W.device
    n_b = N * K // blocksize
    codes = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(n_b, dtype=torch.float32, device=dev)
    aq = torch.empty(n_b, dtype=torch.uint8, device=dev) if double_quant else None
    s2 = torch.empty((n_b + 255) // 256, dtype=torch.float32, device=dev) if double_quant else None
    mu = torch.empty(1, dtype=torch.float32, device=dev) if double_quant else None
    B = torch.empty(N, r, dtype=torch.float32, device=dev)
    A = torch.empty(r, K, dtype=torch.float32, device=dev)
    sigma = torch.empty(r, dtype=torch.float32, device=dev)
    objectives = torch.empty(steps, dtype=torch.float64, device=dev)
    ws_bytes = lib.lq_loftq_workspace(N, K, r, l, int(double_quant))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    P = lambda t: _ptr(t) if t is not None else None
    _check(lib.lq_loftq_init(_ptr(W), N, K, blocksize, int(double_quant), r, l, int(steps), int(power_iters),
                             _ptr(omega), _ptr(codes), _ptr(absmax), P(aq), P(s2), P(mu), _ptr(B), _ptr(A),
                             _ptr(sigma), _ptr(objectives), _ptr(ws), ws_bytes, _stream(dev)), "lq_loftq_init")
    if double_quant:
        qw = QWeight(N, K, codes, absmax_q=aq, dq_scale=s2, dq_mean=mu)
    else:
        qw = QWeight(N, K, codes, absmax=absmax)
    qw.absmax_f32 = absmax
    return qw, B, A, sigma, objectives


class QuantAdapter:
    """A LoRAQuant-quantized adapter: device tensors written by lq_loraquant."""

    def __init__(self, N, K, r, bits_max, device):
        torch = _torch()
        self.N, self.K, self.r = N, K, r
        z = lambda n, dt: torch.empty(n, dtype=dt, device=device)
        self.codes_a = z(r * K * bits_max // 8, torch.uint8)
        self.absmax_a = z(r * K // 64, torch.float32)
        self.codes_b = z(r * N * bits_max // 8, torch.uint8)
        self.absmax_b = z(r * N // 64, torch.float32)
        self.row_bits = z(r, torch.uint8)
        self.offsets_a = z(r + 1, torch.int64)
        self.offsets_b = z(r + 1, torch.int64)
        self.levels_a = z(r * 16, torch.float32)
        self.thresholds_a = z(r * 15, torch.float32)
        self.levels_b = z(r * 16, torch.float32)
        self.thresholds_b = z(r * 15, torch.float32)
        self.sigma = z(r, torch.float32)
        self.h = z(1, torch.int32)
        self.Ap = z(r * K, torch.float32)
        self.Bpt = z(r * N, torch.float32)


def loraquant(B, A, rho: float = 0.9, bits_hi: int = 3, bits_lo: int = 1, h: int = -1) -> QuantAdapter:
    """LoRAQuant-style quantization of B [N, r], A [r, K] (float32, device)."""
    torch = _torch()
    N, r = B.shape
    K = A.shape[1]
    q = QuantAdapter(N, K, r, max(bits_hi, bits_lo), B.device)
    ws_bytes = lib.lq_loraquant_workspace(N, K, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=B.device)
    _check(lib.lq_loraquant(_ptr(B), _ptr(A), N, K, r, float(rho), int(h), int(bits_hi), int(bits_lo),
                            _ptr(q.codes_a), _ptr(q.absmax_a), _ptr(q.codes_b), _ptr(q.absmax_b), _ptr(q.row_bits),
                            _ptr(q.offsets_a), _ptr(q.offsets_b), _ptr(q.levels_a), _ptr(q.thresholds_a),
                            _ptr(q.levels_b), _ptr(q.thresholds_b), _ptr(q.sigma), _ptr(q.h), _ptr(q.Ap),
                            _ptr(q.Bpt), _ptr(ws), ws_bytes, _stream(B.device)),
           "lq_loraquant")
    return q


def loraquant_dequant(q: QuantAdapter):
    """-> (A bf16 [r, K], B bf16 [N, r]) of a quantized adapter."""
    torch = _torch()
    dev = q.codes_a.device
    A = torch.empty(q.r, q.K, dtype=torch.bfloat16, device=dev)
    B = torch.empty(q.N, q.r, dtype=torch.bfloat16, device=dev)
    ws_bytes = lib.lq_loraquant_dequant_workspace(q.N, q.K, q.r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.lq_loraquant_dequant(_ptr(q.codes_a), _ptr(q.absmax_a), _ptr(q.codes_b), _ptr(q.absmax_b),
                                    _ptr(q.row_bits), _ptr(q.offsets_a), _ptr(q.offsets_b), _ptr(q.levels_a),
                                    _ptr(q.levels_b), q.N, q.K, q.r, _ptr(A), _ptr(B), _ptr(ws), ws_bytes,
                                    _stream(dev)),
           "lq_loraquant_dequant")
    return A, B


def quantize_codebook(W, row_bits, thresholds, blocksize: int = 64):
    """W [N, K], row_bits uint8 [N] (device), thresholds f32 [N, 15] (device)
    -> (codes uint8, absmax f32 [N*K/64], row_offset int64 [N+1])."""
    torch = _torch()
    N, K = W.shape
    offs = row_offsets(row_bits.cpu().tolist(), K)
    row_offset = torch.tensor(offs, dtype=torch.int64, device=W.device)
    codes = torch.empty(max(offs[-1], 1), dtype=torch.uint8, device=W.device)
    absmax = torch.empty(N * K // blocksize, dtype=torch.float32, device=W.device)
    _check(lib.lq_quantize_codebook(_ptr(W), _dtype_code(W), N, K, blocksize, _ptr(row_bits), _ptr(row_offset),
                                    _ptr(thresholds), _ptr(codes), _ptr(absmax), _stream(W.device)),
           "lq_quantize_codebook")
    return codes, absmax, row_offset
