// Internal declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lq.h"

// Host-side bounds asserts of the debug build: a failed check reports to
// stderr and the launcher returns hipErrorInvalidValue instead of launching.
#ifdef LQ_DEBUG
#include <cstdio>
#define LQ_DASSERT(cond)                                                                  \
  do {                                                                                    \
    if (!(cond)) {                                                                        \
      std::fprintf(stderr, "lq debug: check failed: %s (%s:%d)\n", #cond, __FILE__, __LINE__); \
      return hipErrorInvalidValue;                                                        \
    }                                                                                     \
  } while (0)
#else
#define LQ_DASSERT(cond) ((void)0)
#endif

namespace lq {

// Block constants of a quantized weight (float32, or double quantized).
struct QConst {
  const float* absmax;
  const uint8_t* absmax_q;
  const float* dq_scale;
  const float* dq_mean;
};

// The 16 NF4 levels (ascending).
struct Nf4Levels {
  float q[16];
};

// Code-search table over 33 bins of width 1/16 covering [-1, 1 + 1/16):
// bin j holds x in [j/16 - 1, (j+1)/16 - 1]. base[j] counts thresholds below
// the bin (with a 2^-20 margin) and T[j] is the one threshold inside the
// widened bin (or 4.0 if there is none), so code(x) = base[j] + (x > T[j]).
struct Nf4Lut {
  float T[33];
  int32_t base[33];
};

// Host-built tables (computed once, then read-only).
struct Tables {
  float levels[16];
  float thresholds[15];
  Nf4Levels lv;
  Nf4Lut lut;
};
const Tables& tables();

// Starting point of the weighted Lloyd-Max learner for widths b = 1..4
// (index b - 1), float64: the NormalFloat levels of width b (2^(b-1) + 1
// quantiles on the positive half, 2^(b-1) on the negative half, the shared 0
// once; {-1, +1} at b = 1) and the midpoints of adjacent levels.
struct LloydInit {
  double L[4][16];
  double T[4][15];
};
const LloydInit& lloyd_init();


// Quantized-weight view used by the kernels.
struct QWeight {
  int32_t format;
  int64_t N, K;
  const uint8_t* codes;
  QConst qc;
  const uint8_t* row_bits;
  const int64_t* row_offset;
  const float* levels;
};

// ---- launchers (return hipError_t of the launch) ----------------------------
hipError_t launch_quantize_nf4(const void* W, int dtype, int64_t n_blocks, uint8_t* codes,
                               float* absmax, hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t n_blocks, uint8_t* absmax_q,
                               float* dq_scale, float* dq_mean, double* ws, hipStream_t s);
size_t double_quant_ws_doubles(int64_t n_blocks);
hipError_t launch_dequant(const QWeight& w, uint16_t* out, hipStream_t s);
// launch_double_quant, then launch_dequant of the NF4 codes with the new
// constants (one kernel after the block sums for up to 1024 DQ blocks).
hipError_t launch_double_quant_dequant(const float* absmax, int64_t n_blocks, uint8_t* absmax_q,
                                      float* dq_scale, float* dq_mean, const uint8_t* codes, uint16_t* out,
                                      double* ws, hipStream_t s);
size_t profile_ws_doubles(int64_t n_blocks);
hipError_t launch_profile_nf4(const void* W, int dtype, int64_t n_blocks, double tau, double* stats,
                              double* ws, hipStream_t s);
hipError_t launch_lloyd(const void* W, int dtype, int64_t N, int64_t K, const uint8_t* row_bits,
                        int max_iters, float* levels, float* thresholds, int32_t* iterations,
                        hipStream_t s);
// Low-rank initialisation (LoftQ-style): building blocks and the alternation.
int lowrank_max_l();
hipError_t launch_lowrank_sub(const float* W, int64_t N, int64_t K, const float* B, const float* A, int r,
                              float* out, hipStream_t s);
hipError_t launch_residual(const float* W, const uint16_t* Wd, int64_t n, float* R, hipStream_t s);
size_t svd_ws_bytes(int64_t N, int64_t K, int l, int r);
hipError_t launch_svd_lowrank(const float* R, int64_t N, int64_t K, int r, int l, int power_iters,
                              const float* omega, float* B, float* A, float* sigma, void* ws, hipStream_t s);
size_t sqerr_ws_bytes();
hipError_t launch_lowrank_sqerr(const float* R, int64_t N, int64_t K, const float* B, const float* A, int r,
                                double* out, void* ws, hipStream_t s);
size_t loftq_ws_bytes(int64_t N, int64_t K, int r, int l, bool dq);
hipError_t launch_loftq(const float* W, int64_t N, int64_t K, bool dq, int r, int l, int steps, int power_iters,
                        const float* omega, uint8_t* codes, float* absmax, uint8_t* absmax_q, float* dq_scale,
                        float* dq_mean, float* B, float* A, float* sigma, double* objectives, void* ws,
                        hipStream_t s);
// LoRAQuant-style adapter quantization.
constexpr int LQ_LORAQUANT_MAX_R = 64;
size_t loraquant_ws_bytes(int64_t N, int64_t K, int r);
hipError_t launch_loraquant(const float* B, const float* A, int64_t N, int64_t K, int r, double rho, int h_fixed,
                            int bits_hi, int bits_lo, uint8_t* codes_a, float* absmax_a, uint8_t* codes_b,
                            float* absmax_b, uint8_t* row_bits, int64_t* offsets_a, int64_t* offsets_b,
                            float* levels_a, float* thresholds_a, float* levels_b, float* thresholds_b,
                            float* sigma, int32_t* h_out, float* Ap_out, float* Bpt_out, void* ws, hipStream_t s);
// Device address of this device's copy of the library's no-allocation
// scratch array (LQ_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t noalloc_scratch(void** out);
// Debug build: read (and optionally clear) the device flag word after a
// device synchronisation; hipErrorNotSupported in the release build.
hipError_t debug_flags(unsigned int* out, bool clear);
hipError_t launch_quantize_codebook(const void* W, int dtype, int64_t N, int64_t K,
                                    const uint8_t* row_bits, const int64_t* row_offset,
                                    const float* thresholds, uint8_t* codes, float* absmax,
                                    hipStream_t s);

// Skinny products. Row form: out[m][j] = sum_c Q[m][c] * R[j][c] with R
// [r, C] row-major (C % 8 == 0); one launch, no workspace. The _rt variant
// (r <= 16) takes the second operand transposed, Rt [C, r] row-major (u = G B).
// With parts > 1 (at most 4) the columns are split into that many ranges and
// out holds their partial sums [parts][M][r], which the consumers add in
// part order; row_skinny_parts(M, C) is the split the layer entry points use.
int row_skinny_parts(int64_t M, int64_t C);
hipError_t launch_row_skinny(const uint16_t* Q, int64_t M, int64_t C, const uint16_t* R, int r,
                             float* out, hipStream_t s, int parts = 1);
hipError_t launch_row_skinny_rt(const uint16_t* Q, int64_t M, int64_t C, const uint16_t* Rt, int r,
                                float* out, hipStream_t s, int parts = 1);
hipError_t launch_transpose_u16(const uint16_t* in, int64_t N, int r, uint16_t* out, hipStream_t s);
// Column form: out(j, c) = scale * sum_m P[m][j] * Q[m][c] with P float32
// [M, r] row-major; written as
// out[j*C + c] (out_transposed = false, [r, C]) or out[c*r + j] ([C, r]).
// launch_col_skinny writes partial sums into ws (col_skinny_ws_floats) and
// describes the reduction that finishes it in *job; launch_reduce_splits2
// runs up to two such reductions in one launch (a job with out == nullptr is
// skipped).
struct SplitJobDesc {
  const float* part = nullptr;
  int splits = 0;
  int64_t rows = 0, cols = 0, srows = 0, pair = 0;
  float scale = 0.0f;
  float* out = nullptr;
  int transposed = 0;
};
size_t col_skinny_ws_floats(int64_t M, int64_t C, int r);
// One column-form product: P [M, r] float32, Q [M, C], its output and
// partial-sum workspace (col_skinny_ws_floats(M, C, r) floats).
struct ColSkinnyReq {
  const float* P;
  const uint16_t* Q;
  int64_t C;
  float scale;
  float* out;
  bool out_transposed;
  float* ws;
};
// Up to two column-form products with the same M and r in one launch
// (either request may be null); fills the reduction job of each.
hipError_t launch_col_skinny(const ColSkinnyReq* a, const ColSkinnyReq* b, int64_t M, int r, SplitJobDesc* ja,
                             SplitJobDesc* jb, hipStream_t s);
hipError_t launch_reduce_splits2(const SplitJobDesc& a, const SplitJobDesc& b, hipStream_t s);

// Dequant-GEMM with the LoRA segment (formed in the kernel from t or u and
// B or A).
//  forward : out[m][n] = sum_k X[m][k] W'[n][k] + s * sum_j t[m][j] B[n][j]
//  backward: out[m][k] = sum_n G[m][n] W'[n][k] + s * sum_j u[m][j] A[j][k]
int lora_seg_cols(int r);
// Workspace of launch_gemm_fwd (fwd) / launch_gemm_bwd: the dequantized bf16
// weight for the codebook format, none for NF4.
size_t gemm_ws_bytes(const QWeight& w, int64_t M, int r, bool fwd);
hipError_t launch_gemm_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype, uint16_t* ws,
                           hipStream_t st);
// With red_a / red_b (may be null), the GEMM's workgroups also run those
// split reductions after their tiles (the partial sums must be complete
// before the launch), which saves the reduction's own launch.
hipError_t launch_gemm_bwd(const QWeight& w, const uint16_t* G, int64_t M, const float* u,
                           const uint16_t* A, int r, float s, uint16_t* gX, uint16_t* ws, hipStream_t st,
                           const SplitJobDesc* red_a = nullptr, const SplitJobDesc* red_b = nullptr);
// The decode GEMV handles NF4 weights whose per-workgroup constant table
// fits in LDS (K <= 33728: one row group of 16 rows); others use the GEMM.
bool gemv_supported(const QWeight& w);
bool gemv_forms_t(const QWeight& w, int64_t M, int r);
// t == nullptr: the kernel forms t = X A^T itself (NF4 weights, r <= 32) and
// writes it to t_out when that is not null; gemv_forms_t says when that is
// the faster choice. t given as t_parts > 1 partial sums: their sum is
// written to t_out when that is not null.
hipError_t launch_gemv_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype,
                           hipStream_t st, const uint16_t* A = nullptr, float* t_out = nullptr,
                           int t_parts = 1);

}  // namespace lq
