#!/usr/bin/env python3
"""Throughput of the quantized-LoRA hot path on one MI355X.

One step = the whole path on the Llama-7B q_proj workload (W 4096x4096
float32 ~ N(0, 0.02^2), 2048 bf16 tokens = batch 4 x seq 512, LoRA r = 16,
alpha = 32): NF4 quantize -> double quantization and dequant to bf16 (one
call) -> forward (one call: t = X A^T, fused dequant-GEMM + LoRA) ->
backward (u, dB, grad_X, dA). Inputs are resident in HBM before timing; four input sets are rotated
so the 256 MB Infinity Cache cannot hold the step's working set.

value = algorithmic GEMM + LoRA flops of the forward and backward per step
divided by the step time (TFLOP/s); quantize / double quant / dequant add time
but no flops. Before the timed window the GPU runs steps for a fixed wall
time (clock settling), then the W warm-up steps.

The JSON line also carries:
  * roofline -- the dominant kernel (the forward dequant-GEMM) timed by HIP
    events around back-to-back launches on rotated inputs (the same kernel
    duration a kernel trace reports), against the bf16 MFMA peak, with its
    HBM traffic from the committed counter profile;
  * kernels -- every kernel of the path on the five workloads (1024^2 latency
    rows, q_proj, the MLP pair, the 1.75-bit codebook layer, decode GEMV),
    each arm run for a fixed wall time after 20 warm-up launches, the median
    of its batches with p10 / p90; memory-bound arms rotate at least 1 GiB
    of distinct buffers so every launch streams from HBM; the forward GEMM
    arm is run twice (replicated arm) and their gap is the noise floor;
  * sessions -- the headline step measured again in fresh processes;
  * cpu_baseline -- the CPU oracle on the host (all BLAS threads, and one).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "dequant-GEMM+LoRA TFLOP/s & quantize/GEMV GB/s; % of MFMA/HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="wall time of untimed steps before the warm-up (clock settling)")
    ap.add_argument("--arm-seconds", type=float, default=0.4, help="wall time of each kernel-table arm")
    ap.add_argument("--sessions", type=int, default=3,
                    help="whole sessions (this process + fresh child processes) of the headline step")
    ap.add_argument("--session-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel table")
    ap.add_argument("--only", default="",
                    help="comma list of kernel-table groups to run (linear1k, q_proj, mlp, lowra, decode); "
                         "default all")
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated through the steps")
    ap.add_argument("--noise-windows", type=int, default=5,
                    help="further timed windows of K steps for the run-to-run spread (0: none)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy 5 times (counter calibration)")
    ap.add_argument("--profile", action="store_true",
                    help="short run for counter collection: no clock settling, spread windows, sessions, "
                         "ceilings or CPU baseline; each kernel arm is 2 warm-up launches and one pass over its "
                         "rotation")
    args = ap.parse_args()
    if args.profile:
        args.settle_seconds, args.noise_windows, args.sessions, args.no_cpu_baseline = 0.0, 0, 1, True
    return args


class Dev:
    """Device copies of one layer's inputs and preallocated outputs."""

    def __init__(self, torch, lq, layer, W, X, A, B, G, M):
        import numpy as np
        dev = torch.device("cuda")
        self.layer, self.M, self.r = layer, M, layer.r
        N, K, r = layer.N, layer.K, layer.r

        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        self.W = torch.from_numpy(W).to(dev)
        self.X = bf(X.bits)
        self.A = bf(A.bits)
        self.B = bf(B.bits)
        self.G = bf(G.bits) if G is not None else None
        n_b = N * K // 64
        n_d = (n_b + 255) // 256
        self.codes = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
        self.absmax = torch.empty(n_b, dtype=torch.float32, device=dev)
        self.aq = torch.empty(n_b, dtype=torch.uint8, device=dev)
        self.s2 = torch.empty(n_d, dtype=torch.float32, device=dev)
        self.mu = torch.empty(1, dtype=torch.float32, device=dev)
        self.stats = torch.empty(2, dtype=torch.float64, device=dev)
        self.prof_ws_bytes = lq.lib.lq_profile_workspace(N, K, 64)
        self.prof_ws = torch.empty(self.prof_ws_bytes, dtype=torch.uint8, device=dev)
        self.dq_ws_bytes = lq.lib.lq_double_quant_workspace(n_b, 256)
        self.dq_ws = torch.empty(self.dq_ws_bytes, dtype=torch.uint8, device=dev)
        self.qw = lq.QWeight(N, K, self.codes, absmax_q=self.aq, dq_scale=self.s2, dq_mean=self.mu)
        self.Wd = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        self.t = torch.empty(M, r, dtype=torch.float32, device=dev)
        self.H = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        self.ld_ws_bytes = lq.lib.lq_lora_down_workspace(M, K, r)
        self.ld_ws = torch.empty(max(self.ld_ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.fw_ws_bytes = lq.lib.lq_dequant_gemm_workspace(self.qw.ref(), M, r)
        self.fw_ws = torch.empty(max(self.fw_ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.qf_ws_bytes = lq.lib.lq_forward_workspace(self.qw.ref(), M, r)
        self.qf_ws = torch.empty(max(self.qf_ws_bytes, 1), dtype=torch.uint8, device=dev)
        if G is not None:
            self.gX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
            self.dA = torch.empty(r, K, dtype=torch.float32, device=dev)
            self.dB = torch.empty(N, r, dtype=torch.float32, device=dev)
            self.u = torch.empty(M, r, dtype=torch.float32, device=dev)
            self.bw_ws_bytes = lq.lib.lq_backward_workspace(self.qw.ref(), M, r)
            self.bw_ws = torch.empty(self.bw_ws_bytes, dtype=torch.uint8, device=dev)
            self.gx_ws_bytes = lq.lib.lq_dequant_gemm_t_workspace(self.qw.ref(), M, r)
            self.gx_ws = torch.empty(max(self.gx_ws_bytes, 1), dtype=torch.uint8, device=dev)


class Calls:
    """The library entry points bound to one Dev's buffers (raw C-ABI calls)."""

    def __init__(self, torch, lq, d: Dev):
        self.lq, self.d = lq, d
        self.lib = lq.lib
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        self.P = P
        L = d.layer
        self.alpha = float(L.alpha)
        self.args_q = (P(d.W), 0, L.N, L.K, 64, P(d.codes), P(d.absmax), self.stream)
        self.args_prof = (P(d.W), 0, L.N, L.K, 64, ctypes.c_double(0.01), P(d.stats), P(d.prof_ws),
                          d.prof_ws_bytes, self.stream)
        self.args_dq = (P(d.absmax), L.N * L.K // 64, 256, P(d.aq), P(d.s2), P(d.mu), P(d.dq_ws),
                        d.dq_ws_bytes, self.stream)
        self.args_deq = (d.qw.ref(), P(d.Wd), self.stream)
        self.args_dqd = (P(d.absmax), L.N * L.K // 64, 256, P(d.aq), P(d.s2), P(d.mu), P(d.codes), P(d.Wd),
                         P(d.dq_ws), d.dq_ws_bytes, self.stream)
        self.args_ld = (P(d.X), d.M, L.K, P(d.A), d.r, P(d.t), P(d.ld_ws), d.ld_ws_bytes, self.stream)
        self.args_fwd = (d.qw.ref(), P(d.X), d.M, P(d.t), P(d.B), d.r, self.alpha, P(d.H), 1,
                         P(d.fw_ws), d.fw_ws_bytes, self.stream)
        self.args_qfwd = (d.qw.ref(), P(d.X), d.M, P(d.A), P(d.B), d.r, self.alpha, P(d.H), 1, P(d.t),
                          P(d.qf_ws), d.qf_ws_bytes, self.stream)
        if d.G is not None:
            self.args_bwd = (d.qw.ref(), P(d.X), P(d.G), d.M, P(d.A), P(d.B), d.r, self.alpha, P(d.t),
                             P(d.gX), P(d.dA), P(d.dB), P(d.bw_ws), d.bw_ws_bytes, self.stream)
            self.args_gx = (d.qw.ref(), P(d.G), d.M, P(d.u), P(d.A), d.r, self.alpha, P(d.gX),
                            P(d.gx_ws), d.gx_ws_bytes, self.stream)

    def chk(self, st, name):
        if st != 0:
            raise RuntimeError(f"{name} failed: {st}")

    def profile(self):
        self.chk(self.lib.lq_profile_nf4(*self.args_prof), "profile")

    def quantize(self):
        self.chk(self.lib.lq_quantize_nf4(*self.args_q), "quantize")

    def double_quant(self):
        self.chk(self.lib.lq_double_quant(*self.args_dq), "double_quant")

    def dequant(self):
        self.chk(self.lib.lq_dequant(*self.args_deq), "dequant")

    def double_quant_dequant(self):
        self.chk(self.lib.lq_double_quant_dequant(*self.args_dqd), "double_quant_dequant")

    def lora_down(self):
        self.chk(self.lib.lq_lora_down(*self.args_ld), "lora_down")

    def fwd_gemm(self):
        self.chk(self.lib.lq_dequant_gemm(*self.args_fwd), "dequant_gemm")

    def qlora_forward(self):
        self.chk(self.lib.lq_qlora_forward(*self.args_qfwd), "qlora_forward")

    def backward(self):
        self.chk(self.lib.lq_qlora_backward(*self.args_bwd), "backward")

    def grad_x(self):
        self.chk(self.lib.lq_dequant_gemm_t(*self.args_gx), "dequant_gemm_t")

    def step(self, ev=None):
        """One pass of the path; `ev` = (start, end) events put around the
        forward call (t = X A^T, then the dequant-GEMM) on the same stream."""
        self.quantize()
        self.double_quant_dequant()
        if ev is not None:
            ev[0].record()
        self.qlora_forward()
        if ev is not None:
            ev[1].record()
        self.backward()


def make_devs(torch, lq, syn, name, n_sets, M=None, with_grad=True):
    import numpy as np
    L = syn.LAYERS[name]
    M = L.M if M is None else M
    W = syn.weight(L)
    X = syn.activations(L, M)
    A, B = syn.lora_a(L), syn.lora_b(L)
    G = syn.grad_out(L, M) if with_grad else None
    devs = [Dev(torch, lq, L, W, X, A, B, G, M)]
    for k in range(1, n_sets):
        # extra copies (distinct buffers, same values) defeat the Infinity Cache
        devs.append(Dev(torch, lq, L, W, X, A, B, G, M))
    return devs


def kernel_event_stride(steps):
    """Steps between the timed steps whose forward call gets its own
    event pair: every 4th, or closer so that at least 5 calls are timed."""
    return max(1, min(4, steps // 5))


ARM_WARMUP = 20
PROFILE_ARMS = False   # set by --profile: arms of 2 warm-ups and one pass over the rotation


def time_arm(torch, fns, seconds, warmup=ARM_WARMUP):
    """One fixed-duration arm: `warmup` untimed launches, then batches of
    back-to-back launches of fns[i % len(fns)] (each batch about 20 ms,
    bracketed by HIP events on the current stream, which is the stream the
    library launches on) until `seconds` of wall time have passed (at least
    3 batches). Returns (median, p10, p90) ms per launch over the batches and
    the number of timed launches."""
    n = len(fns)
    if PROFILE_ARMS:
        for i in range(2):
            fns[i % n]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k = max(n, 3)
        e0.record()
        for i in range(k):
            fns[i % n]()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / k
        return ms, ms, ms, k
    for i in range(warmup):
        fns[i % n]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # calibration batch: one pass over the rotation (at least 4 launches)
    cal = n * max(1, -(-4 // n))
    e0.record()
    for i in range(cal):
        fns[i % n]()
    e1.record()
    e1.synchronize()
    est = max(e0.elapsed_time(e1) / cal, 1e-3)
    batch = max(1, int(round(20.0 / est / n))) * n
    per, k, launches = [], 0, 0
    t0 = time.perf_counter()
    while len(per) < 3 or time.perf_counter() - t0 < seconds:
        e0.record()
        for i in range(batch):
            fns[(k + i) % n]()
        e1.record()
        e1.synchronize()
        per.append(e0.elapsed_time(e1) / batch)
        k += batch
        launches += batch
    per.sort()
    pick = lambda q: per[min(len(per) - 1, int(round(q * (len(per) - 1))))]
    return pick(0.5), pick(0.1), pick(0.9), launches


def time_ms(torch, fns, seconds):
    return time_arm(torch, fns, seconds)[0]


def layer_flops(L, M):
    N, K, r = L.N, L.K, L.r
    fwd_gemm = 2 * M * N * K + 2 * M * N * r
    lora_down = 2 * M * K * r
    bwd = 2 * M * N * K + 4 * M * r * (N + K)
    gx = 2 * M * N * K + 2 * M * K * r
    return {"fwd_gemm": fwd_gemm, "lora_down": lora_down, "fwd": fwd_gemm + lora_down, "bwd": bwd, "grad_x": gx}


def codec_bytes(L, M=0):
    n = L.N * L.K
    n_b = n // 64
    n_d = (n_b + 255) // 256
    packed = n // 2 + n_b + 4 * n_d + 4
    return {
        "quantize": 4 * n + n // 2 + 4 * n_b,
        "profile": 4 * n,
        "double_quant": 4 * n_b + n_b + 4 * n_d + 4,
        "dequant": packed + 2 * n,
        "double_quant_dequant": 4 * n_b + n // 2 + n_b + 4 * n_d + 4 + 2 * n,
        "gemv": packed + 2 * L.K * M + 2 * L.N * L.r + 2 * L.N * M + 4 * M * L.r,
    }


def rec_loraquant(torch, lq, name, d, rec, kernels, arm_s, rho=0.9, bits_hi=3, bits_lo=1):
    """LoRAQuant-style quantization of the layer's adapter (float32 copies of
    its bf16 B [N, r] and A [r, K]): time per call and the adapter's error."""
    import numpy as np
    N, r = d.B.shape
    K = d.A.shape[1]
    B32, A32 = d.B.float().contiguous(), d.A.float().contiguous()
    q = lq.QuantAdapter(N, K, r, max(bits_hi, bits_lo), B32.device)
    wsb = lq.lib.lq_loraquant_workspace(N, K, r)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        if lq.lib.lq_loraquant(P(B32), P(A32), N, K, r, rho, -1, bits_hi, bits_lo, P(q.codes_a), P(q.absmax_a),
                               P(q.codes_b), P(q.absmax_b), P(q.row_bits), P(q.offsets_a), P(q.offsets_b),
                               P(q.levels_a), P(q.thresholds_a), P(q.levels_b), P(q.thresholds_b), P(q.sigma),
                               P(q.h), P(q.Ap), P(q.Bpt), P(ws), wsb, st) != 0:
            raise RuntimeError("lq_loraquant failed")
    # reads B and A, writes the float32 reparameterized factors and reads them
    # twice (codebook learner, quantizer), writes codes and constants
    byts = 4 * r * (N + K) + 12 * r * (N + K) + r * (N + K) * bits_hi // 8 + 4 * r * (N + K) // 64
    rec(f"{name}.loraquant", time_arm(torch, [run], arm_s), byts, "GB/s")
    Ad, Bd = lq.loraquant_dequant(q)
    ref = B32.double() @ A32.double()
    err = ((Bd.double() @ Ad.double() - ref).norm() / ref.norm()).item()
    kernels[f"{name}.loraquant"].update({"h": int(q.h.item()), "rel_error": round(err, 4), "r": r,
                                         "bits_hi": bits_hi, "bits_lo": bits_lo, "rho": rho})


def loftq_bytes(L, r, q, steps):
    """Algorithmic bytes of the LoftQ-style initialisation: per alternation,
    W - B A (read W, write it; skipped in the first), NF4 quantize + double
    quant + dequant, the residual (read W and W', write R), the rank-r SVD
    (2 q + 3 passes over R for the tall-skinny products) and the error sum
    (one more pass); the small l x l work is not counted."""
    n = L.N * L.K
    n_b = n // 64
    quant = 4 * n + n // 2 + 4 * n_b
    dqb = 4 * n_b + n_b + 4 * ((n_b + 255) // 256) + 4
    deq = n // 2 + n_b + 2 * n
    resid = 4 * n + 2 * n + 4 * n
    svd = (2 * q + 3) * 4 * n
    sq = 4 * n
    per = quant + dqb + deq + resid + svd + sq
    return steps * per + (steps - 1) * 8 * n


def lowra_bytes(syn, L):
    """Algorithmic bytes of the per-channel codebook kernels: the learner reads
    W and writes levels, thresholds and iteration counts; the quantizer reads
    W, the widths, offsets and thresholds and writes the bit planes and the
    block constants."""
    import numpy as np
    n = L.N * L.K
    bits = syn.lowra_row_bits(L).astype(np.int64)
    planes = int(np.sum(L.K * bits // 8))
    n_b = n // 64
    weight = planes + n_b + 4 * ((n_b + 255) // 256) + 4 + L.N + 8 * (L.N + 1) + L.N * 16 * 4
    return {
        "lloyd": 4 * n + L.N + L.N * (16 + 15 + 1) * 4,
        "quantize": 4 * n + L.N + 8 * (L.N + 1) + L.N * 15 * 4 + planes + 4 * (n // 64),
        # decode GEMV: the double-quantized codebook weight (planes, E4M3
        # constants, scales, mean, widths, offsets, levels) + X, t, B in, H out
        "gemv": lambda M: weight + 2 * L.K * M + 4 * M * L.r + 2 * L.N * L.r + 2 * L.N * M,
        "weight": weight,
    }


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "dq_gemm_fwd_q_proj_traffic.md")
TRAFFIC_SOURCES = ("quantized_lora_fine_lq_amd/csrc/lq_gemm.hip", "quantized_lora_fine_lq_amd/csrc/lq_device.h")


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the forward dequant-GEMM, from the committed
    FETCH_SIZE / WRITE_SIZE counter runs (calibrated on a plain copy), or
    None if the kernel sources changed since those counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    vals = {}
    for ln in lines:
        if ln.startswith("traffic_bytes_per_launch:") or ln.startswith("source_digest:"):
            k, v = ln.split(":", 1)
            vals[k] = v.strip()
    if vals.get("source_digest") != kernel_source_digest() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def cpu_baseline(syn):
    """The oracle (numpy / float64 BLAS) on whole q_proj steps, repeated
    until about 10 s of CPU work, on all the BLAS threads; then its forward +
    backward on a 512-token slice of the same step on one thread."""
    import numpy as np
    from oracle import nf4, dq, layer
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
        cores = os.cpu_count() or 1
    L = syn.LAYERS["q_proj"]
    W, X, A, B, G = syn.weight(L), syn.activations(L), syn.lora_a(L), syn.lora_b(L), syn.grad_out(L)
    times = []
    # whole q_proj steps until about 10 s of CPU work (at least 3 steps)
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 200):
        t0 = time.perf_counter()
        packed, c = nf4.quantize(W)
        code8, s2, mu = dq.double_quant(c)
        Wd = nf4.dequant(packed, dq.dq_decode(code8, s2, mu), W.shape)
        H, t = layer.forward(Wd, X.f32, A.f32, B.f32, L.alpha)
        dX, dA, dB = layer.backward(Wd, X.f32, G.f32, A.f32, B.f32, L.alpha)
        times.append(time.perf_counter() - t0)
    total = sum(times)
    fl = layer_flops(L, L.M)
    out = {"value": round(len(times) * (fl["fwd"] + fl["bwd"]) / total / 1e12, 4), "unit": "TFLOP/s",
           "cores": int(cores), "kind": "oracle", "seconds": round(total, 2),
           "seconds_per_step_median": round(sorted(times)[len(times) // 2], 3),
           "sample": f"{len(times)} full q_proj steps (quantize, double quant, dequant, float64 forward + "
                     f"backward) on the host CPU, {total:.1f} s in all; value = their flops / that time"}
    if threadpool_limits is not None:
        Ms = 512
        Xs, Gs = X.f32[:Ms], G.f32[:Ms]
        with threadpool_limits(limits=1):
            reps = []
            while len(reps) < 2 or (sum(reps) < 3.0 and len(reps) < 20):
                t0 = time.perf_counter()
                layer.forward(Wd, Xs, A.f32, B.f32, L.alpha)
                layer.backward(Wd, Xs, Gs, A.f32, B.f32, L.alpha)
                reps.append(time.perf_counter() - t0)
        fls = layer_flops(L, Ms)
        out["single_thread"] = {
            "value": round(len(reps) * (fls["fwd"] + fls["bwd"]) / sum(reps) / 1e12, 4), "unit": "TFLOP/s",
            "cores": 1, "sample": f"{len(reps)} float64 forward + backward passes over the first {Ms} of the "
                                  f"step's {L.M} tokens, one BLAS thread, {sum(reps):.1f} s"}
    return out


def copy_ceiling_gbs(torch) -> float:
    """Measured memory ceiling: torch's own device copy of 1 GiB (1 GiB read
    + 1 GiB written per copy), HIP events around 5 copies after 2 warm-ups."""
    src = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbs = 5 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def sclk_under_load(torch, step) -> dict | None:
    """The shader clock while the step runs: about a second of steps is
    queued, then rocm-smi (a separate process reading the driver's clock
    report) samples the current sclk. None when the tool is missing or its
    output has no sclk line."""
    import re
    import shutil
    import subprocess
    tool = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi" if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if tool is None:
        return None
    for _ in range(3000):
        step()
    try:
        r = subprocess.run([tool, "--showclocks"], capture_output=True, text=True, timeout=30)
        txt = r.stdout
    except Exception:
        txt = ""
    torch.cuda.synchronize()
    m = re.search(r"sclk[^\n]*?\((\d+)\s*Mhz\)", txt, re.IGNORECASE)
    if not m:
        return None
    return {"MHz": int(m.group(1)), "how": "rocm-smi --showclocks while ~1 s of q_proj steps was queued"}


class CodecSet:
    """Distinct buffers for the memory-bound codec arms of one layer: a copy
    of W and every output of quantize, the profiling pass, double quant and
    dequant."""

    def __init__(self, torch, lq, L, W_dev):
        dev = torch.device("cuda")
        N, K = L.N, L.K
        n_b = N * K // 64
        n_d = (n_b + 255) // 256
        self.N, self.K = N, K
        self.W = W_dev.clone()
        self.codes = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
        self.absmax = torch.empty(n_b, dtype=torch.float32, device=dev)
        self.aq = torch.empty(n_b, dtype=torch.uint8, device=dev)
        self.s2 = torch.empty(n_d, dtype=torch.float32, device=dev)
        self.mu = torch.empty(1, dtype=torch.float32, device=dev)
        self.stats = torch.empty(2, dtype=torch.float64, device=dev)
        self.prof_b = lq.lib.lq_profile_workspace(N, K, 64)
        self.prof_ws = torch.empty(self.prof_b, dtype=torch.uint8, device=dev)
        self.dq_b = lq.lib.lq_double_quant_workspace(n_b, 256)
        self.dq_ws = torch.empty(self.dq_b, dtype=torch.uint8, device=dev)
        self.Wd = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        self.qw = lq.QWeight(N, K, self.codes, absmax_q=self.aq, dq_scale=self.s2, dq_mean=self.mu)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        lib = lq.lib
        n = N * K

        def chk(v, name):
            if v != 0:
                raise RuntimeError(f"{name} failed: {v}")
        self.quantize = lambda: chk(lib.lq_quantize_nf4(P(self.W), 0, N, K, 64, P(self.codes), P(self.absmax), st),
                                    "quantize")
        self.profile = lambda: chk(lib.lq_profile_nf4(P(self.W), 0, N, K, 64, ctypes.c_double(0.01), P(self.stats),
                                                      P(self.prof_ws), self.prof_b, st), "profile")
        self.double_quant = lambda: chk(lib.lq_double_quant(P(self.absmax), n // 64, 256, P(self.aq), P(self.s2),
                                                            P(self.mu), P(self.dq_ws), self.dq_b, st), "double_quant")
        self.dequant = lambda: chk(lib.lq_dequant(self.qw.ref(), P(self.Wd), st), "dequant")
        self.double_quant_dequant = lambda: chk(lib.lq_double_quant_dequant(
            P(self.absmax), n // 64, 256, P(self.aq), P(self.s2), P(self.mu), P(self.codes), P(self.Wd),
            P(self.dq_ws), self.dq_b, st), "double_quant_dequant")


def rotation_count(n_weights, min_bytes=1 << 30):
    """Copies such that one pass over them moves at least `min_bytes` in the
    smallest of the rotated codec arms (dequant: 2.5 B per weight)."""
    return max(1, -(-min_bytes // (5 * n_weights // 2)))


def codec_sets(torch, lq, L, W_dev, min_bytes=1 << 30):
    """rotation_count(N K) CodecSets of one layer, quantized once."""
    sets = [CodecSet(torch, lq, L, W_dev) for _ in range(rotation_count(L.N * L.K, min_bytes))]
    for c in sets:
        c.quantize()
        c.double_quant()
    torch.cuda.synchronize()
    return sets


def run_sessions(args):
    """The headline step again in fresh processes (started before this
    process touches the GPU); returns their ms per step."""
    import subprocess
    out = []
    for _ in range(max(0, args.sessions - 1)):
        cmd = [sys.executable, os.path.abspath(__file__), "--session-child", "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--settle-seconds", str(args.settle_seconds), "--sets", str(args.sets)]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        if r.returncode != 0:
            raise RuntimeError(f"session child failed ({r.returncode}): {r.stderr[-2000:]}")
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]
        out.append(json.loads(line)["ms_per_step"])
        log(f"session child: {out[-1]:.5f} ms/step")
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the quantized-LoRA hot path here is a single-GPU "
              "kernel library, and sharding across GPUs is a design note, not a run.", flush=True)
        sys.exit(2)
    child_ms = [] if args.session_child else run_sessions(args)
    global PROFILE_ARMS
    PROFILE_ARMS = args.profile
    import numpy as np
    import torch
    import quantized_lora_fine_lq_amd as lq
    import synthetic as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log("generating q_proj inputs")
    devs = make_devs(torch, lq, syn, "q_proj", args.sets)
    calls = [Calls(torch, lq, d) for d in devs]
    L = syn.LAYERS["q_proj"]
    fl = layer_flops(L, L.M)
    step_flops = fl["fwd"] + fl["bwd"]
    arm_s = args.arm_seconds

    if args.copy_probe:
        # plain copy of known size: 512 MiB read + 512 MiB written per launch
        src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- clock settling, warm-up, the timed step --------------------------
    # Steps for a fixed wall time first: the shader clock rises over the
    # first second or so of load, and a count-only warm-up can end before it
    # has (the first window then runs slower than the later ones).
    settle_steps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_seconds:
        for i in range(50):
            calls[(settle_steps + i) % len(calls)].step()
        settle_steps += 50
        torch.cuda.synchronize()
    settle = {"seconds": round(time.perf_counter() - t0, 3), "steps": settle_steps}
    for i in range(args.warmup):
        calls[i % len(calls)].step()
    torch.cuda.synchronize()
    # the forward call inside the timed steps also gets event pairs
    # (every ev_stride-th step: each pair adds a few microseconds to its step)
    ev_stride = kernel_event_stride(args.steps)
    kev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in range(0, args.steps, ev_stride)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        calls[i % len(calls)].step(kev.get(i))
    e1.record()
    e1.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    value = step_flops / (ms_step * 1e-3) / 1e12
    log(f"step: {ms_step:.4f} ms  ({value:.1f} TFLOP/s), wall {wall:.3f} s, settle {settle}")
    if args.session_child:
        print(json.dumps({"ms_per_step": ms_step}), flush=True)
        return

    # run-to-run spread: further windows of the same K steps, after the
    # headline window (which alone gives value and ms_per_step)
    windows = []
    for w in range(args.noise_windows):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for i in range(args.steps):
            calls[(i + w) % len(calls)].step()
        a1.record()
        a1.synchronize()
        windows.append(a0.elapsed_time(a1) / args.steps)
    spread = None
    pick = lambda v, q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    if windows:
        ws = sorted(windows)
        spread = {"windows": len(ws), "steps_each": args.steps, "ms_per_step_p10": round(pick(ws, 0.1), 5),
                  "ms_per_step_p50": round(pick(ws, 0.5), 5), "ms_per_step_p90": round(pick(ws, 0.9), 5)}
        log("spread", spread)
    sess = sorted([ms_step] + child_ms)
    sessions = {"count": len(sess), "ms_per_step": [round(x, 5) for x in [ms_step] + child_ms],
                "median": round(pick(sess, 0.5), 5),
                "spread_frac": round((sess[-1] - sess[0]) / pick(sess, 0.5), 4),
                "how": "headline window of this process and of fresh child processes (same arguments)"}

    # ---- dominant kernel: forward dequant-GEMM on q_proj -------------------
    # Two arms of back-to-back launches over the rotated input sets: the
    # first gives the roofline, the replicated second the noise floor.
    f1 = time_arm(torch, [c.fwd_gemm for c in calls], arm_s)
    f2 = time_arm(torch, [c.fwd_gemm for c in calls], arm_s)
    fwd_ms = f1[0]
    fwd_tflops = fl["fwd_gemm"] / (fwd_ms * 1e-3) / 1e12
    in_step_ms = sum(a.elapsed_time(b) for a, b in kev.values()) / len(kev)
    roofline = {"bound": "mfma", "kernel": "k_dq_gemm<ProdFwdNF4<true>> (q_proj, M=2048)",
                "achieved": round(fwd_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(fwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(),
                "avg_us": round(fwd_ms * 1e3, 2), "p10_us": round(f1[1] * 1e3, 2), "p90_us": round(f1[2] * 1e3, 2),
                "launches_timed": f1[3],
                "how": "HIP events around batches of back-to-back launches on the library's stream, "
                       f"{len(calls)} input sets rotated, {ARM_WARMUP} warm-up launches, median batch",
                "replicated_arm_us": round(f2[0] * 1e3, 2),
                "noise_floor": round(abs(f1[0] - f2[0]) / (0.5 * (f1[0] + f2[0])), 4),
                "in_step_forward_call_us": round(in_step_ms * 1e3, 2), "in_step_calls": len(kev),
                "in_step_note": "events around the whole lq_qlora_forward call inside timed steps "
                                "(t = X A^T, then this GEMM)",
                "algorithmic_flop_per_launch": fl["fwd_gemm"]}
    log("roofline", roofline)

    kernels = {}
    ceilings = None
    only = set(x for x in args.only.split(",") if x)
    want = lambda g: not only or g in only
    if not args.no_kernels:
        copy_gbs = 5000.0 if args.profile else copy_ceiling_gbs(torch)
        if not args.profile:
            ceilings = {"copy_GB/s": round(copy_gbs, 1),
                        "copy": "torch device copy, 1 GiB read + 1 GiB written; frac_copy in the kernel table is "
                                "relative to it",
                        "sclk": sclk_under_load(torch, calls[0].step)}
            log("ceilings", ceilings)

        def rec(name, arm, work, unit, rotated=None):
            ms, p10, p90, n = arm
            k = {"us": round(ms * 1e3, 2), "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
                 "launches": n}
            if unit == "GB/s":
                ach = work / (ms * 1e-3) / 1e9
                k.update({"GB/s": round(ach, 1), "frac_hbm": round(ach / HBM_PEAK_GBS, 4),
                          "frac_copy": round(ach / copy_gbs, 4), "bytes": work})
            elif unit == "TFLOP/s":
                ach = work / (ms * 1e-3) / 1e12
                k.update({"TFLOP/s": round(ach, 1), "frac_mfma": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "flop": work})
            else:
                k["bound"] = "latency (time only)"
            if rotated is not None:
                k["rotated_bytes"] = int(rotated)
            kernels[name] = k
            log(name, k)

        rec("q_proj.dequant_gemm_fwd", f1, fl["fwd_gemm"], "TFLOP/s")
        rec("q_proj.dequant_gemm_fwd#replicate", f2, fl["fwd_gemm"], "TFLOP/s")

        if want("linear1k"):
            # BASELINE's first workload: 1024 x 1024, 16 tokens -- latency rows
            L1 = syn.LAYERS["linear1k"]
            d1 = make_devs(torch, lq, syn, "linear1k", 1, with_grad=False)
            c1 = Calls(torch, lq, d1[0])
            c1.quantize(); c1.double_quant(); c1.lora_down()
            rec("linear1k.quantize_nf4", time_arm(torch, [c1.quantize], arm_s), None, "us")
            rec("linear1k.double_quant", time_arm(torch, [c1.double_quant], arm_s), None, "us")
            rec("linear1k.dequant", time_arm(torch, [c1.dequant], arm_s), None, "us")
            rec("linear1k.lora_down", time_arm(torch, [c1.lora_down], arm_s), None, "us")
            rec("linear1k.dequant_gemm_fwd", time_arm(torch, [c1.fwd_gemm], arm_s), None, "us")
            # the whole forward in one call (at 16 tokens the GEMV forms t itself)
            rec("linear1k.qlora_forward", time_arm(torch, [c1.qlora_forward], arm_s), None, "us")
            del c1, d1

        if want("q_proj"):
            cb = codec_bytes(L)
            cs = codec_sets(torch, lq, L, devs[0].W)
            rot = lambda b: b * len(cs)
            rec("q_proj.quantize_nf4", time_arm(torch, [c.quantize for c in cs], arm_s), cb["quantize"], "GB/s",
                rot(cb["quantize"]))
            rec("q_proj.profile_nf4", time_arm(torch, [c.profile for c in cs], arm_s), cb["profile"], "GB/s",
                rot(cb["profile"]))
            rec("q_proj.double_quant", time_arm(torch, [c.double_quant for c in cs], arm_s), cb["double_quant"], "GB/s",
                rot(cb["double_quant"]))
            rec("q_proj.dequant", time_arm(torch, [c.dequant for c in cs], arm_s), cb["dequant"], "GB/s",
                rot(cb["dequant"]))
            rec("q_proj.double_quant_dequant", time_arm(torch, [c.double_quant_dequant for c in cs], arm_s),
                cb["double_quant_dequant"], "GB/s", rot(cb["double_quant_dequant"]))
            del cs
            torch.cuda.empty_cache()
            rec("q_proj.lora_down", time_arm(torch, [c.lora_down for c in calls], arm_s), fl["lora_down"], "TFLOP/s")
            for c in calls:
                c.lora_down()
            rec("q_proj.backward", time_arm(torch, [c.backward for c in calls], arm_s), fl["bwd"], "TFLOP/s")

            # LoftQ-style initialisation of the q_proj adapter (r = 16, l = 32, 8 power steps, 5 alternations)
            r_lq, l_lq, q_lq, t_lq = L.r, 2 * L.r, 8, 5
            d0 = devs[0]
            om = torch.from_numpy(np.random.default_rng(1).standard_normal((L.K, l_lq)).astype(np.float32)).cuda()
            Bq = torch.empty(L.N, r_lq, dtype=torch.float32, device="cuda")
            Aq = torch.empty(r_lq, L.K, dtype=torch.float32, device="cuda")
            sg = torch.empty(r_lq, dtype=torch.float32, device="cuda")
            ob = torch.empty(t_lq, dtype=torch.float64, device="cuda")
            lws_b = lq.lib.lq_loftq_workspace(L.N, L.K, r_lq, l_lq, 1)
            lws = torch.empty(lws_b, dtype=torch.uint8, device="cuda")
            P = lambda t: ctypes.c_void_p(t.data_ptr())
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

            def loftq():
                if lq.lib.lq_loftq_init(P(d0.W), L.N, L.K, 64, 1, r_lq, l_lq, t_lq, q_lq, P(om), P(d0.codes),
                                        P(d0.absmax), P(d0.aq), P(d0.s2), P(d0.mu), P(Bq), P(Aq), P(sg), P(ob),
                                        P(lws), lws_b, st) != 0:
                    raise RuntimeError("lq_loftq_init failed")
            rec("q_proj.loftq_init", time_arm(torch, [loftq], arm_s, warmup=2), loftq_bytes(L, r_lq, q_lq, t_lq),
                "GB/s")
            kernels["q_proj.loftq_init"]["objectives"] = [round(x, 4) for x in ob.cpu().tolist()]
            del lws
            rec_loraquant(torch, lq, "q_proj", d0, rec, kernels, arm_s)
        del calls, devs
        torch.cuda.empty_cache()

        if want("mlp"):
            for name in ("mlp_up", "mlp_down"):
                log(f"generating {name} inputs")
                Lm = syn.LAYERS[name]
                dv = make_devs(torch, lq, syn, name, 2)
                cs = [Calls(torch, lq, d) for d in dv]
                for c in cs:
                    c.quantize(); c.double_quant(); c.lora_down()
                flm = layer_flops(Lm, Lm.M)
                qs = codec_sets(torch, lq, Lm, dv[0].W)
                cbm = codec_bytes(Lm)
                rec(f"{name}.quantize_nf4", time_arm(torch, [c.quantize for c in qs], arm_s), cbm["quantize"], "GB/s",
                    cbm["quantize"] * len(qs))
                rec(f"{name}.dequant", time_arm(torch, [c.dequant for c in qs], arm_s), cbm["dequant"], "GB/s",
                    cbm["dequant"] * len(qs))
                del qs
                torch.cuda.empty_cache()
                rec(f"{name}.dequant_gemm_fwd", time_arm(torch, [c.fwd_gemm for c in cs], arm_s), flm["fwd_gemm"],
                    "TFLOP/s")
                rec(f"{name}.backward", time_arm(torch, [c.backward for c in cs], arm_s), flm["bwd"], "TFLOP/s")
                if name == "mlp_up":
                    rec_loraquant(torch, lq, name, dv[0], rec, kernels, arm_s)
                del cs, dv
                torch.cuda.empty_cache()

        if want("lowra"):
            # ---- per-channel codebook layer (LowRA): learner, quantizer, GEMM ----
            log("generating lowra inputs")
            Ll = syn.LAYERS["lowra"]
            lb = lowra_bytes(syn, Ll)
            Wl = torch.from_numpy(syn.weight(Ll)).cuda()
            bits_h = syn.lowra_row_bits(Ll)
            bl = torch.from_numpy(bits_h).cuda()
            P = lambda t: ctypes.c_void_p(t.data_ptr())
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            lv = torch.empty(Ll.N, 16, dtype=torch.float32, device="cuda")
            th = torch.empty(Ll.N, 15, dtype=torch.float32, device="cuda")
            its = torch.empty(Ll.N, dtype=torch.int32, device="cuda")

            def lloyd():
                if lq.lib.lq_lloyd_codebooks(P(Wl), 0, Ll.N, Ll.K, 64, P(bl), 100, P(lv), P(th), P(its), st) != 0:
                    raise RuntimeError("lq_lloyd_codebooks failed")
            rec("lowra.lloyd_codebooks", time_arm(torch, [lloyd], arm_s, warmup=2), lb["lloyd"], "GB/s")
            kernels["lowra.lloyd_codebooks"]["iterations_mean"] = round(its.float().mean().item(), 2)
            kernels["lowra.lloyd_codebooks"]["iterations_max"] = int(its.max().item())
            offs = lq.row_offsets(bits_h.tolist(), Ll.K)
            roff = torch.tensor(offs, dtype=torch.int64, device="cuda")
            n_rot = max(1, -(-(1 << 30) // lb["quantize"]))
            rot_sets = [(Wl.clone(), torch.empty(offs[-1], dtype=torch.uint8, device="cuda"),
                         torch.empty(Ll.N * Ll.K // 64, dtype=torch.float32, device="cuda")) for _ in range(n_rot)]

            def cb_quant(ws):
                Wc, cc, am = ws
                if lq.lib.lq_quantize_codebook(P(Wc), 0, Ll.N, Ll.K, 64, P(bl), P(roff), P(th), P(cc), P(am), st) != 0:
                    raise RuntimeError("lq_quantize_codebook failed")
            rec("lowra.quantize_codebook", time_arm(torch, [(lambda ws=ws: cb_quant(ws)) for ws in rot_sets], arm_s),
                lb["quantize"], "GB/s", lb["quantize"] * n_rot)
            del rot_sets
            qwl = lq.QWeight.from_codebook(Wl, bl, th, lv)
            Xl, Al, Bl = syn.activations(Ll), syn.lora_a(Ll), syn.lora_b(Ll)
            bfd = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
            Xd, Ad, Bd = bfd(Xl.bits), bfd(Al.bits), bfd(Bl.bits)
            tl = torch.empty(Ll.M, Ll.r, dtype=torch.float32, device="cuda")
            lq.lora_down(Xd, Ad, tl)
            Hl = torch.empty(Ll.M, Ll.N, dtype=torch.bfloat16, device="cuda")
            flw = layer_flops(Ll, Ll.M)
            rec("lowra.dequant_gemm_fwd",
                time_arm(torch, [lambda: lq.dequant_gemm(qwl, Xd, tl, Bd, Ll.alpha, out=Hl)], arm_s),
                flw["fwd_gemm"], "TFLOP/s")
            # decode GEMV over copies of the codebook weight (>= 1 GiB per pass)
            n_cp = max(1, -(-(1 << 30) // lb["weight"]))
            cb_copies = [qwl] + [lq.QWeight(Ll.N, Ll.K, qwl.codes.clone(), absmax_q=qwl.absmax_q.clone(),
                                            dq_scale=qwl.dq_scale.clone(), dq_mean=qwl.dq_mean.clone(),
                                            fmt=lq.LQ_FMT_CODEBOOK, row_bits=bl, row_offset=qwl.row_offset,
                                            levels=lv) for _ in range(n_cp - 1)]
            for M in (1, 16):
                Hm = torch.empty(M, Ll.N, dtype=torch.bfloat16, device="cuda")
                Xm, tm = Xd[:M].contiguous(), tl[:M].contiguous()
                fns = [(lambda q=q: lq.dequant_gemm(q, Xm, tm, Bd, Ll.alpha, out=Hm)) for q in cb_copies]
                gb = lb["gemv"](M)
                rec(f"lowra.gemv_M{M}", time_arm(torch, fns, arm_s), gb, "GB/s", gb * len(cb_copies))
            del cb_copies
            del Wl, qwl, Xd, Hl
            torch.cuda.empty_cache()

        if want("decode"):
            log("generating decode inputs")
            Ld = syn.LAYERS["decode"]
            dv = make_devs(torch, lq, syn, "decode", 1, M=16, with_grad=False)
            c0 = Calls(torch, lq, dv[0])
            cbd = codec_bytes(Ld)
            ds = codec_sets(torch, lq, Ld, dv[0].W)
            rec("decode.quantize_nf4", time_arm(torch, [c.quantize for c in ds], arm_s), cbd["quantize"], "GB/s",
                cbd["quantize"] * len(ds))
            rec("decode.profile_nf4", time_arm(torch, [c.profile for c in ds], arm_s), cbd["profile"], "GB/s",
                cbd["profile"] * len(ds))
            rec("decode.double_quant", time_arm(torch, [c.double_quant for c in ds], arm_s), cbd["double_quant"],
                "GB/s", cbd["double_quant"] * len(ds))
            rec("decode.dequant", time_arm(torch, [c.dequant for c in ds], arm_s), cbd["dequant"], "GB/s",
                cbd["dequant"] * len(ds))
            del ds
            c0.quantize(); c0.double_quant()
            # 9 copies of the 121 MB quantized weight rotate through the GEMV
            copies = [dv[0].qw]
            keep = []
            for k in range(8):
                cc = dv[0].codes.clone(); aq = dv[0].aq.clone(); s2 = dv[0].s2.clone(); mu = dv[0].mu.clone()
                keep.append((cc, aq, s2, mu))
                copies.append(lq.QWeight(Ld.N, Ld.K, cc, absmax_q=aq, dq_scale=s2, dq_mean=mu))
            del dv[0].W
            torch.cuda.empty_cache()
            for M in (1, 4, 16):
                X = dv[0].X[:M].contiguous()
                t = torch.zeros(M, Ld.r, dtype=torch.float32, device="cuda")
                lq.lora_down(X, dv[0].A, t)
                H = torch.empty(M, Ld.N, dtype=torch.bfloat16, device="cuda")
                fns = [(lambda q=q: lq.dequant_gemm(q, X, t, dv[0].B, Ld.alpha, out=H)) for q in copies]
                gb = codec_bytes(Ld, M)["gemv"]
                rec(f"decode.gemv_M{M}", time_arm(torch, fns, arm_s), gb, "GB/s", gb * len(copies))

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "q_proj 4096x4096 NF4 + double quant, 2048 tokens (batch 4 x seq 512), "
                               "LoRA r=16 alpha=32; step = quantize + double quant + dequant + forward + backward",
                   "global_batch": L.M, "tokens": L.M, "N": L.N, "K": L.K, "r": L.r, "alpha": L.alpha,
                   "input_sets_rotated": args.sets},
        "roofline": roofline,
        "settle": settle,
        "step_spread": spread,
        "sessions": sessions,
        "cpu_baseline": None,
        "ceilings": ceilings,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on q_proj steps")
        out["cpu_baseline"] = cpu_baseline(syn)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
