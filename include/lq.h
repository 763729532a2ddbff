/*
 * lq.h -- C ABI of the MI355X (gfx950) quantized-LoRA hot path.
 *
 * The operations follow these pages:
 *   [QLoRA]  Heng's Blog, "QLoRA: Efficient Finetuning of Quantized LLMs":
 *            the layer equation (introduction), NF4 (section "Contribution 1:
 *            4-bit NormalFloat (NF4)"), double quantization (section
 *            "Contribution 2: Double Quantization").
 *   [LowRA]  cloud.tencent.com.cn write-up of LowRA: per-output-channel
 *            quantization with custom thresholds and a given precision
 *            (section 3, workflow; section 4.1 and figure 3).
 *
 * Conventions (every entry point):
 *   - Tensors are dense row-major. W is [N, K] (out x in, the Linear
 *     convention), X is [M, K], A is [r, K], B is [N, r], H and G are [M, N].
 *   - All tensor pointers are DEVICE pointers allocated and owned by the
 *     caller. The library never allocates or frees device memory and holds no
 *     mutable global state; it is safe to call from several host threads.
 *   - Scratch memory is a caller-provided device workspace whose size comes
 *     from the matching *_workspace() query.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Every call is asynchronous on that stream and never synchronizes.
 *   - bfloat16 data is passed as uint16_t bit patterns.
 *   - Every call returns an lq_status. Arguments are validated before anything
 *     is launched; on an error nothing is launched and outputs are untouched.
 *     No C++ exception crosses this boundary.
 *   - Alignment (checked: a misaligned pointer returns LQ_ERR_ARG before any
 *     launch). Bulk tensors are moved with 16-byte vector accesses and must be
 *     16-byte aligned: codes (NF4 and codebook) and absmax_q of a weight
 *     descriptor, X, G, A, B, a bfloat16 H, grad_X, the lq_dequant output,
 *     every workspace, and the float32 matrices of the low-rank entry points
 *     (W, out, R, omega, B, A, Ap, Bpt). W of lq_quantize_nf4 and
 *     lq_profile_nf4 needs 16 bytes for float32 and 8 for bfloat16 / float16;
 *     the codes output of lq_quantize_nf4 needs 8. Arrays accessed element by
 *     element need only their natural alignment: absmax, dq_scale, dq_mean,
 *     t, u, dA, dB, a float32 H, stats, levels, thresholds, sigma,
 *     objectives (4 or 8 bytes), row_offset (8). lq_quantize_codebook and
 *     lq_lloyd_codebooks read W element by element where it is not 16-byte
 *     aligned, so any element-aligned W is accepted there. Rows stay aligned
 *     because K % 64 == 0 (K % 8 == 0 for lq_lora_down).
 *   - Preconditions not checked in the release build: inputs are finite;
 *     codebook thresholds are strictly increasing per row; row_offset holds
 *     the prefix sums of K*b/8; device pointers are valid and large enough for
 *     the stated sizes. Violations give undefined results. The LQ_DEBUG build
 *     (liblq_debug.so, same entry points) checks the codebook tables on the
 *     host before launching and records non-finite weights and non-increasing
 *     thresholds seen by the quantizers in a device flag word
 *     (lq_debug_flags below).
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum lq_status {
  LQ_OK = 0,
  LQ_ERR_ARG = -1,          /* null or misaligned pointer, bad enum value */
  LQ_ERR_SHAPE = -2,        /* K % 64 != 0, r outside [1, 128], sizes <= 0 */
  LQ_ERR_UNSUPPORTED = -3,  /* blocksize != 64, dq blocksize != 256, dtype */
  LQ_ERR_WORKSPACE = -4,    /* workspace missing or too small */
  LQ_ERR_LAUNCH = -5        /* the HIP runtime reported an error at launch */
};

/* ---- element types ----------------------------------------------------- */
enum lq_dtype { LQ_F32 = 0, LQ_BF16 = 1, LQ_F16 = 2 };

/* ---- quantized weight formats ------------------------------------------ */
enum lq_format {
  LQ_FMT_NF4 = 0,       /* 4-bit NF4 codes, two per byte, high nibble first */
  LQ_FMT_CODEBOOK = 1   /* per-row b-bit codes as bit-planes (see below) */
};

/*
 * Descriptor of a quantized frozen weight W [N, K] (plain pointers, no
 * ownership). The 64-element quantization blocks run along K, so block j of
 * row i covers W[i, 64j .. 64j+63] and its flat index is i*(K/64) + j.
 *
 * Block constants, one of:
 *   absmax != NULL : float32 constant per block [N*K/64];
 *   absmax == NULL : double-quantized constants -- absmax_q [N*K/64] (OCP
 *                    E4M3 codes), dq_scale [ceil(N*K/64 / 256)] float32 and
 *                    dq_mean [1] float32; the constant of block j is
 *                    fma(E4M3(absmax_q[j]), dq_scale[j / 256], dq_mean[0]).
 *
 * LQ_FMT_NF4: codes [N*K/2] bytes; byte e/2 holds flat element e (even) in
 *   bits 7..4 and element e+1 in bits 3..0.
 * LQ_FMT_CODEBOOK: row i has row_bits[i] = b in {1,2,3,4}; its bytes start at
 *   codes + row_offset[i] (row_offset[N+1], row_offset[0] = 0,
 *   row_offset[i+1] - row_offset[i] = K*b/8). Each 64-block of the row is b
 *   little-endian uint64 bit-planes; bit e of plane p is bit p of the code of
 *   the block's element e. levels [N, 16] float32 holds the row's mapping
 *   (first 2^b entries used); the dequantized weight is
 *   bfloat16(float32(levels[i, code] * constant)).
 */
typedef struct lq_qweight {
  int32_t format;          /* lq_format */
  int32_t blocksize;       /* must be 64 */
  int64_t N;
  int64_t K;
  const uint8_t* codes;
  const float* absmax;
  const uint8_t* absmax_q;
  const float* dq_scale;
  const float* dq_mean;
  int32_t dq_blocksize;    /* must be 256 when double quantized */
  int32_t reserved0;       /* set to 0 */
  const uint8_t* row_bits;   /* LQ_FMT_CODEBOOK only */
  const int64_t* row_offset; /* LQ_FMT_CODEBOOK only */
  const float* levels;       /* LQ_FMT_CODEBOOK only */
} lq_qweight;

/* Storage of one quantized [N, K] weight ([QLoRA] Contribution 2). */
typedef struct lq_sizes_t {
  int64_t n;                    /* N*K */
  int64_t n_blocks;             /* N*K/64 */
  int64_t n_dq_blocks;          /* ceil(n_blocks/256) */
  int64_t code_bytes;           /* N*K*bits/8 (NF4: bits = 4) */
  int64_t dq_const_bytes;       /* n_blocks + 4*n_dq_blocks + 4 */
  int64_t fp32_const_bytes;     /* 4*n_blocks */
  double const_bits_per_param_dq;   /* 8/64 + 32/(64*256) = 0.126953125 */
  double const_bits_per_param_fp32; /* 32/64 = 0.5 */
} lq_sizes_t;

/* Static description of a status code. Never NULL. */
const char* lq_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int lq_version(void);

/*
 * Host-side NF4 tables ([QLoRA] Contribution 1). levels[16]: the 16 NF4 values
 * in ascending order, float32 (q0 = -1, q7 = +0, q15 = +1): 8 negative-half and
 * 9 positive-half standard-normal quantiles at equal probability steps from
 * 1/2 to delta = 1 - (1/32 + 1/30)/2, scaled by 1/Phi^-1(delta), duplicate 0
 * dropped. thresholds[15]: t_i = largest float32 <= (q_i + q_{i+1})/2, so that
 * code = #{i : x > t_i} is the nearest level with ties to the lower index.
 * Either pointer may be NULL. Pure host function; needs no GPU.
 */
int lq_nf4_table(float* levels, float* thresholds);

/*
 * Size arithmetic for an [N, K] weight quantized at `bits` bits per weight
 * (4 for NF4; 1..4 for a uniform codebook). Pure host function.
 * LQ_ERR_SHAPE if N <= 0, K <= 0 or K % 64 != 0; LQ_ERR_ARG if out is NULL or
 * bits is outside 1..4.
 */
int lq_sizes(int64_t N, int64_t K, int32_t bits, lq_sizes_t* out);

/*
 * Blockwise NF4 quantization ([QLoRA] Contribution 1): for each 64-block j,
 * absmax[j] = max |w| (float32); x = w / absmax[j] (IEEE float32 division,
 * x = +0 for an all-zero block); code = #{i : x > t_i}; codes packed two per
 * byte as described for LQ_FMT_NF4.
 *   W        [N, K] of `dtype` (LQ_F32, LQ_BF16 or LQ_F16; bf16/f16 are widened
 *            exactly to float32 first)
 *   codes    [N*K/2] bytes, written
 *   absmax   [N*K/64] float32, written
 * Errors: LQ_ERR_ARG (null pointer, bad dtype), LQ_ERR_SHAPE (N, K <= 0,
 * K % 64 != 0), LQ_ERR_UNSUPPORTED (blocksize != 64), LQ_ERR_LAUNCH.
 */
int lq_quantize_nf4(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize,
                    uint8_t* codes, float* absmax, void* stream);

/* Workspace bytes for lq_profile_nf4: 16 bytes per 64 weight blocks. */
size_t lq_profile_workspace(int64_t N, int64_t K, int32_t blocksize);

/*
 * AQLoRA profiling pass ([AQLoRA] section 3.1): for one layer's weight
 * W [N, K] (dtype LQ_F32 / LQ_BF16 / LQ_F16, bf16 and f16 converted exactly),
 * flattened into 64-blocks as in lq_quantize_nf4,
 *   stats[0] = eps = (1/|W|) * sum over blocks of ||b - NF4^-1(NF4(b))||_2^2
 *   stats[1] = s   = fraction of weights with |w| < tau (exact comparison)
 * The round trip uses the float32 block constant and the float32 product
 * level * constant; each squared error is formed in float64 and the sum is
 * reduced in a fixed order (the result is reproducible run to run).
 *   stats  device double [2], written
 *   workspace  device memory of lq_profile_workspace(N, K, 64) bytes
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE (K % 64 != 0, sizes <= 0),
 * LQ_ERR_UNSUPPORTED (blocksize != 64), LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_profile_nf4(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize, double tau,
                   double* stats, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_double_quant (float64 partial sums). */
size_t lq_double_quant_workspace(int64_t n_blocks, int32_t dq_blocksize);

/*
 * Double quantization of the block constants ([QLoRA] Contribution 2): the
 * mean mu of all n_blocks constants (float64 sum as a fixed binary tree --
 * pairwise within each 256-constant block, then pairwise over the block sums
 * padded with zeros to a power of two -- divided by n_blocks, rounded to
 * float32) is subtracted; for each 256-block J, a2 = max |c - mu|,
 * dq_scale[J] = a2 / 448 (float32), and each constant is stored as the OCP
 * E4M3 code (round to nearest even) of clamp((c - mu) / dq_scale[J], -448, 448)
 * (code 0 when dq_scale[J] == 0). The last block may be partial.
 *   absmax    [n_blocks] float32, read
 *   absmax_q  [n_blocks] E4M3 codes, written
 *   dq_scale  [ceil(n_blocks/256)] float32, written
 *   dq_mean   [1] float32, written
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE (n_blocks <= 0), LQ_ERR_UNSUPPORTED
 * (dq_blocksize != 256), LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_double_quant(const float* absmax, int64_t n_blocks, int32_t dq_blocksize,
                    uint8_t* absmax_q, float* dq_scale, float* dq_mean,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * Dequantization to bfloat16 ([QLoRA] introduction: dequantized to BFloat16 at
 * use time): out[i, k] = bfloat16_rne(float32(level(code) * constant)).
 *   w    quantized weight descriptor (NF4 or codebook)
 *   out  [N, K] bfloat16, written
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_LAUNCH.
 */
int lq_dequant(const lq_qweight* w, uint16_t* out, void* stream);

/*
 * Double quantization followed by dequantization to bfloat16, in one call:
 * the results of lq_double_quant on absmax, then of lq_dequant on the NF4
 * weight whose packed codes are `codes` with the new double-quantized
 * constants ([QLoRA] Contribution 2, and the introduction's dequantization
 * to BFloat16). Up to 1024 double-quantization blocks (262144 constants,
 * 16.7 M weights) the encoder and the dequantization are one kernel: each
 * workgroup encodes 256 constants and dequantizes the 16384 weights they
 * scale, so the constants are not read back. Larger weights run the two
 * calls' kernels in turn.
 *   absmax, absmax_q, dq_scale, dq_mean, workspace  as lq_double_quant
 *     (workspace: lq_double_quant_workspace bytes)
 *   codes [n_blocks * 32] packed NF4 codes (two per byte, first code in the
 *         high nibble), read; out [n_blocks * 64] bfloat16, written (the
 *         weight's row-major element order)
 *   codes and out 16-byte aligned
 * Errors: as lq_double_quant.
 */
int lq_double_quant_dequant(const float* absmax, int64_t n_blocks, int32_t dq_blocksize,
                            uint8_t* absmax_q, float* dq_scale, float* dq_mean, const uint8_t* codes,
                            uint16_t* out, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_qlora_forward with M tokens and rank r. */
size_t lq_forward_workspace(const lq_qweight* w, int64_t M, int32_t r);

/*
 * QLoRA forward ([QLoRA] introduction): with W' the bfloat16 dequantized
 * weight and s = alpha / r,
 *     t = X A^T            (float32, [M, r])
 *     H = X W'^T + s t B^T (float32 accumulation, stored as h_dtype)
 * For an NF4 weight W' is never materialised in memory: packed codes are
 * dequantized inside the GEMM (M <= 16 and K <= 33728 use the memory-bound
 * GEMV kernel, other shapes the MFMA GEMM; the environment variable
 * LQ_FORCE_PATH=gemm selects the GEMM at any M, a testing aid); for r <= 32
 * the GEMV forms t itself, so the whole forward is one launch. A codebook
 * weight at M <= 16 (K <= 32576) goes through its own GEMV kernel, which
 * reads the bit-planes directly; at other shapes it is first dequantized
 * into the workspace by its per-channel dequantization kernel ([LowRA]
 * section 3), then multiplied by the MFMA GEMM.
 *   X  [M, K] bf16;  A [r, K] bf16;  B [N, r] bf16
 *   H  [M, N] of h_dtype (LQ_BF16 or LQ_F32), written
 *   t_save [M, r] float32, written if not NULL (for the backward)
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE (M <= 0, r outside [1, 128]),
 * LQ_ERR_UNSUPPORTED (h_dtype), LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_qlora_forward(const lq_qweight* w, const uint16_t* X, int64_t M,
                     const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                     void* H, int32_t h_dtype, float* t_save,
                     void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_lora_down: 0 (no workspace is needed; the
 * workspace arguments of lq_lora_down are ignored and may be NULL / 0). */
size_t lq_lora_down_workspace(int64_t M, int64_t K, int32_t r);

/*
 * First stage of the forward ([QLoRA] introduction, the A x term):
 * t = X A^T in float32.
 *   X [M, K] bf16, A [r, K] bf16, t [M, r] float32 (written).
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE (M, K <= 0, K % 8 != 0, r outside
 * [1, 128]), LQ_ERR_LAUNCH.
 */
int lq_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int32_t r, float* t,
                 void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_dequant_gemm with M tokens and rank r: on the GEMM
 * path, N * K * 2 bytes (rounded up to 256) for the dequantized weight of a
 * codebook weight, plus 256 KB of float32 partial sums per split output
 * tile. The GEMM runs one 256 x 128 output tile per workgroup, one per CU,
 * over 8 XCDs of 32 CUs, each XCD a contiguous range of tiles; when an XCD's
 * last round would be at most half full (and K >= 1024), its last tiles are
 * split into two halves of the contraction and a second launch adds them
 * (e.g. M = 4096, N = 11008, K = 4096: 96 split tiles, 24 MiB). 0 for a
 * weight on the GEMV path and for NF4 shapes that split nothing (the
 * kernels form the LoRA-segment operands themselves). */
size_t lq_dequant_gemm_workspace(const lq_qweight* w, int64_t M, int32_t r);

/*
 * Second stage of the forward ([QLoRA] introduction): given t = X A^T,
 * H = X W'^T + (alpha / r) t B^T with W' dequantized inside the kernel (the
 * GEMV kernels for M <= 16, else the MFMA GEMM, as for lq_qlora_forward; on
 * the GEMM path a codebook weight is dequantized into the workspace first). Arguments as lq_qlora_forward;
 * t [M, r] float32 is read. The workspace (caller-owned,
 * lq_dequant_gemm_workspace bytes) receives the dequantized codebook weight
 * and the split tiles' partial sums; it may be NULL when that size is 0.
 */
int lq_dequant_gemm(const lq_qweight* w, const uint16_t* X, int64_t M, const float* t,
                    const uint16_t* B, int32_t r, float alpha, void* H, int32_t h_dtype,
                    void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_dequant_gemm_t: N * K * 2 (rounded up to 256) for a
 * codebook weight, plus the split tiles' partial sums as for
 * lq_dequant_gemm (output tiles of grad_X [M, K], contraction over N). */
size_t lq_dequant_gemm_t_workspace(const lq_qweight* w, int64_t M, int32_t r);

/*
 * The transposed dequant-GEMM of the backward ([QLoRA] introduction: the
 * gradient flows through the frozen 4-bit base): given u = G B,
 * grad_X = G W' + (alpha / r) u A, bfloat16 output.
 *   G [M, N] bf16, u [M, r] float32, A [r, K] bf16, grad_X [M, K] bf16.
 * NF4 weights are dequantized inside the GEMM, codebook weights into the
 * workspace first. N % 8 == 0 (LQ_ERR_SHAPE); workspace of
 * lq_dequant_gemm_t_workspace bytes (LQ_ERR_WORKSPACE; NULL allowed when 0).
 */
int lq_dequant_gemm_t(const lq_qweight* w, const uint16_t* G, int64_t M, const float* u,
                      const uint16_t* A, int32_t r, float alpha, uint16_t* grad_X,
                      void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_qlora_backward with M tokens and rank r. */
size_t lq_backward_workspace(const lq_qweight* w, int64_t M, int32_t r);

/*
 * QLoRA backward ([QLoRA] introduction: gradients flow through the frozen
 * 4-bit base into the adapter; W gets none). With G = dL/dH and s = alpha/r:
 *     u      = G B               (float32 [M, r], internal)
 *     dB     = s G^T t           [N, r] float32
 *     grad_X = G W' + s u A      [M, K] bf16
 *     dA     = s u^T X           [r, K] float32
 *   G [M, N] bf16; X [M, K] bf16 (needed for dA and when t_saved is NULL)
 *   t_saved [M, r] float32 from the forward, or NULL to recompute t = X A^T
 *   grad_X, dA, dB may each be NULL to skip that output.
 * Requires N % 8 == 0 (LQ_ERR_SHAPE). For a codebook weight, grad_X
 * dequantizes it into the workspace first. The workspace
 * (lq_backward_workspace bytes) holds u, t when recomputed, B^T when
 * r > 16, and partial sums (the column-form products' and, for grad_X, the
 * split tiles' as for lq_dequant_gemm_t); the
 * call sets up whatever it needs, so its contents on entry do not matter.
 * Errors: as lq_qlora_forward.
 */
int lq_qlora_backward(const lq_qweight* w, const uint16_t* X, const uint16_t* G, int64_t M,
                      const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                      const float* t_saved, uint16_t* grad_X, float* dA, float* dB,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * Per-output-channel codebook quantization ([LowRA] section 3: a quantization
 * kernel with custom thresholds and a given precision per output channel;
 * section 4.1: groups of 64 scaled by their absmax). For row i with
 * b = row_bits[i]: absmax and x as in lq_quantize_nf4; code = #{k < 2^b - 1 :
 * x > thresholds[i, k]}; packed as bit-planes as described for
 * LQ_FMT_CODEBOOK.
 *   W           [N, K] of dtype
 *   row_bits    [N] uint8 in {1, 2, 3, 4}
 *   row_offset  [N + 1] int64 byte offsets (prefix sums of K*b/8)
 *   thresholds  [N, 15] float32, first 2^b - 1 of each row used, increasing
 *   codes       [row_offset[N]] bytes, written
 *   absmax      [N*K/64] float32, written
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_LAUNCH.
 */
int lq_quantize_codebook(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize,
                         const uint8_t* row_bits, const int64_t* row_offset,
                         const float* thresholds, uint8_t* codes, float* absmax, void* stream);

/* Limits of lq_lloyd_codebooks: row length (one row is sorted in the LDS of
 * one workgroup) and iteration count. */
#define LQ_LLOYD_MAX_K 16384
#define LQ_LLOYD_MAX_ITERS_LIMIT 100000

/*
 * Weighted Lloyd-Max learner for per-output-channel codebooks ([LowRA]
 * section 5, mapping and threshold learner), for use with
 * lq_quantize_codebook. For each row i of W [N, K] with b = row_bits[i] in
 * {1, 2, 3, 4} (values outside are clamped into that range):
 *   data x = w / c (float32, exactly as lq_quantize_nf4 normalises), weight c
 *   (the absmax of the element's 64-block);
 *   start: thresholds = midpoints of the NormalFloat levels of width b (2^(b-1)
 *   + 1 normal quantiles on the positive half, 2^(b-1) on the negative half,
 *   equal probability steps up to delta_b = 1 - (1/(2 * 2^b) + 1/(2 (2^b - 1)))/2,
 *   the shared 0 once; {-1, +1} at b = 1), levels = those NormalFloat levels;
 *   iteration: code = number of thresholds below x; level j = sum(c x)/sum(c)
 *   over code j (an empty code keeps its level); error = sum(c (x - level)^2)
 *   / sum(c); thresholds = midpoints of adjacent levels;
 *   stop after max_iters iterations or after the first iteration whose error
 *   is not below the previous one; the last computed levels are the result.
 * All learner arithmetic is float64; the interval sums are formed in a fixed
 * order, so results repeat exactly run to run.
 *   W           [N, K] of dtype (LQ_F32, LQ_BF16, LQ_F16; widened exactly)
 *   row_bits    [N] uint8, device
 *   max_iters   1 .. LQ_LLOYD_MAX_ITERS_LIMIT (100 in the method)
 *   levels      [N, 16] float32, written: the first 2^b are the levels rounded
 *               to nearest float32, the rest repeat the last one
 *   thresholds  [N, 15] float32, written: the first 2^b - 1 are the largest
 *               float32 not above the midpoint of adjacent float32 levels
 *               (so lq_quantize_codebook maps x to its nearest level, ties
 *               to the lower one), the rest 3.0
 *   iterations  [N] int32, written (may be NULL): iterations computed per row
 * Errors: LQ_ERR_ARG (null pointer, bad dtype, max_iters out of range),
 * LQ_ERR_SHAPE (N, K <= 0, K % 64 != 0, N > 2^31 - 1), LQ_ERR_UNSUPPORTED
 * (blocksize != 64, K > LQ_LLOYD_MAX_K), LQ_ERR_LAUNCH.
 */
int lq_lloyd_codebooks(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize,
                       const uint8_t* row_bits, int32_t max_iters, float* levels,
                       float* thresholds, int32_t* iterations, void* stream);

/*
 * Low-rank initialisation of the adapter ([LowRA] sections 3 and 5: LoftQ,
 * five alternating steps in which the weight minus the current adapter is
 * quantized and the adapter is refit to what quantization leaves).
 *
 * lq_lowrank_sub: out = float32(W - B A), the rank-r product summed in
 * float64 in order j = 0 .. r-1 (each product of two float32 values is exact
 * there) and subtracted from W in float64 before the single rounding.
 *   W, out [N, K] float32 (out may alias W); B [N, r], A [r, K] float32;
 *   16-byte aligned, K % 4 == 0. r = 0 copies W.
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE (sizes <= 0, K % 4 != 0, r outside [0, 128]),
 * LQ_ERR_LAUNCH.
 */
int lq_lowrank_sub(const float* W, int64_t N, int64_t K, const float* B, const float* A, int32_t r,
                   float* out, void* stream);

/*
 * lq_residual: R = float32(W - W') elementwise, W' a bfloat16 weight (for
 * example lq_dequant's output): what the quantized base misses.
 *   W, R [n] float32 (16-byte aligned), Wd [n] bfloat16 (8-byte aligned), n % 4 == 0.
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_LAUNCH.
 */
int lq_residual(const float* W, const uint16_t* Wd, int64_t n, float* R, void* stream);

/* Workspace bytes for lq_svd_lowrank (0 for an invalid shape). */
size_t lq_svd_lowrank_workspace(int64_t N, int64_t K, int32_t r, int32_t l);

/*
 * Rank-r SVD of R [N, K] (float32, row-major, 16-byte aligned, K % 4 == 0), split evenly between the
 * factors: B = U_r S_r^(1/2) [N, r], A = S_r^(1/2) V_r^T [r, K], sigma = the r
 * largest singular values [r], so that B A approximates the best rank-r
 * approximation of R. Computed by randomized subspace iteration on l >= r
 * columns: Y = R omega, then power_iters steps of Z = R^T Y, Y = R Z, every
 * block orthonormalised (Cholesky QR applied twice, float64 Gram); then the
 * Rayleigh-Ritz step on Z = R^T Y (eigenvectors of Z^T Z by cyclic Jacobi in
 * float64). The result approaches the truncated SVD as power_iters grows; its
 * error is the part of the spectrum the iteration has not separated (see the
 * tests for the measured gap to the exact SVD). Deterministic for a given
 * omega (all reductions in a fixed order).
 *   omega  [K, l] float32, caller-drawn (standard normal is the usual choice)
 *   l      even, r <= l <= min(N, K, 96) (LQ_ERR_SHAPE; above 96 LQ_ERR_UNSUPPORTED)
 *   power_iters 0 .. 1000 (LQ_ERR_ARG)
 *   B [N, r], A [r, K], sigma [r] float32, written
 * A numerically rank-deficient R gives zero factors and sigma = 0 past its rank.
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_svd_lowrank(const float* R, int64_t N, int64_t K, int32_t r, int32_t l, int32_t power_iters,
                   const float* omega, float* B, float* A, float* sigma, void* workspace, size_t ws_bytes,
                   void* stream);

/* Workspace bytes for lq_loftq_init (0 for an invalid shape). */
size_t lq_loftq_workspace(int64_t N, int64_t K, int32_t r, int32_t l, int32_t double_quant);

/*
 * LoftQ-style initialisation ([LowRA] sections 3 and 5). Starting from
 * B = 0, A = 0, each of `steps` alternations
 *   Q   = NF4 quantization of W - B A (lq_lowrank_sub, then lq_quantize_nf4 and,
 *         if double_quant, lq_double_quant),
 *   R   = W - W' with W' the bf16 dequantized Q (lq_dequant, lq_residual),
 *   B,A = rank-r SVD of R (lq_svd_lowrank with l, power_iters, omega),
 * and optionally objectives[t] = ||R - B A||_F^2 (float64, fixed-order sum):
 * the error the adapter leaves after step t.
 * The outputs are the last step's quantized weight (codes, absmax and, with
 * double_quant, absmax_q / dq_scale / dq_mean, laid out as lq_quantize_nf4 and
 * lq_double_quant write them) and the float32 factors B [N, r], A [r, K].
 *   W  [N, K] float32, K % 64 == 0; blocksize 64; steps 1 .. 100 (5 in the method)
 *   objectives [steps] device float64, may be NULL
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_loftq_init(const float* W, int64_t N, int64_t K, int32_t blocksize, int32_t double_quant, int32_t r,
                  int32_t l, int32_t steps, int32_t power_iters, const float* omega, uint8_t* codes,
                  float* absmax, uint8_t* absmax_q, float* dq_scale, float* dq_mean, float* B, float* A,
                  float* sigma, double* objectives, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_loraquant (0 for an invalid shape). */
size_t lq_loraquant_workspace(int64_t N, int64_t K, int32_t r);

/*
 * LoRAQuant-style mixed-precision quantization of a LoRA adapter ([LoRAQuant]
 * method overview and key design). For B [N, r] and A [r, K] (float32,
 * row-major):
 *   reparameterization by the SVD of B A, split evenly: B' = U S^(1/2),
 *   A' = S^(1/2) V^T (computed from the r x r Grams B^T B and A A^T in float64,
 *   so that B' A' = B A and B'^T B' = A' A'^T = diag(sigma)); component i =
 *   row i of A' and column i of B', signed so that the largest-magnitude
 *   entry of row i of A' (the first on ties) is positive;
 *   h = the given h if h >= 0, else the smallest count whose squared float32
 *   singular values, summed in order, reach rho times their total (0 for a
 *   zero adapter);
 *   components i < h quantized at bits_hi, the rest at bits_lo, each vector
 *   (row of A', row of B'^T) in the codebook format of lq_quantize_codebook
 *   with its own codebook from the weighted Lloyd-Max learner
 *   (lq_lloyd_codebooks, 100 iterations at most) at its width.
 * Outputs (device, caller-owned):
 *   codes_a  bytes of A' [r, K]: up to r K bits_max / 8; absmax_a [r K / 64]
 *   codes_b  bytes of B'^T [r, N]: up to r N bits_max / 8; absmax_b [r N / 64]
 *   row_bits [r] uint8; offsets_a, offsets_b [r + 1] int64 (byte offsets)
 *   levels_a, levels_b [r, 16], thresholds_a, thresholds_b [r, 15] float32
 *               (the learned tables of A' rows and B'^T rows)
 *   sigma [r] float32 (descending), h_out [1] int32
 *   Ap [r, K], Bpt [r, N] float32 reparameterized factors (may be NULL)
 * Requires N % 64 == 0, K % 64 == 0 (LQ_ERR_SHAPE), r <= 64 and N, K <=
 * LQ_LLOYD_MAX_K (LQ_ERR_UNSUPPORTED), widths 1..4 and h <= r (LQ_ERR_ARG).
 * Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED, LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_loraquant(const float* B, const float* A, int64_t N, int64_t K, int32_t r, double rho, int32_t h,
                 int32_t bits_hi, int32_t bits_lo, uint8_t* codes_a, float* absmax_a, uint8_t* codes_b,
                 float* absmax_b, uint8_t* row_bits, int64_t* offsets_a, int64_t* offsets_b, float* levels_a,
                 float* thresholds_a, float* levels_b, float* thresholds_b, float* sigma, int32_t* h_out, float* Ap,
                 float* Bpt, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes for lq_loraquant_dequant (N * r * 2). */
size_t lq_loraquant_dequant_workspace(int64_t N, int64_t K, int32_t r);

/*
 * The quantized adapter back in bfloat16 for the layer: A_bf16 [r, K] and
 * B_bf16 [N, r] (row-major), each value bfloat16(level * absmax) as
 * lq_dequant computes it for a codebook weight. Arguments as written by
 * lq_loraquant. Errors: LQ_ERR_ARG, LQ_ERR_SHAPE, LQ_ERR_UNSUPPORTED,
 * LQ_ERR_WORKSPACE, LQ_ERR_LAUNCH.
 */
int lq_loraquant_dequant(const uint8_t* codes_a, const float* absmax_a, const uint8_t* codes_b,
                         const float* absmax_b, const uint8_t* row_bits, const int64_t* offsets_a,
                         const int64_t* offsets_b, const float* levels_a, const float* levels_b, int64_t N,
                         int64_t K, int32_t r, uint16_t* A_bf16, uint16_t* B_bf16, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * lq_qlora_backward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and errors as
 * lq_qlora_backward minus the workspace; its scratch is a library-owned
 * device array of LQ_NOALLOC_SCRATCH_BYTES per GPU (reserved on every GPU
 * the library runs on until the process ends). Shapes whose backward
 * workspace (lq_qlora_backward_noalloc_bytes, equal to lq_backward_workspace)
 * exceeds that size are refused with LQ_ERR_WORKSPACE before anything runs:
 * the NF4 layers of the 4096 x 4096 / 2048-token and 4096 <-> 11008 /
 * 4096-token (r = 64) workloads fit. The call allocates nothing and never
 * synchronizes (the LQ_DEBUG build's layout check of codebook weights
 * aside). All calls on one GPU share its array, which keeps the last call's
 * contents (the call writes every piece before reading it): calls that may
 * overlap on one GPU -- on different streams, or from several host threads
 * -- race on it and must be serialised by the caller.
 */
#define LQ_NOALLOC_SCRATCH_BYTES (96u << 20)
size_t lq_qlora_backward_noalloc_bytes(const lq_qweight* w, int64_t M, int32_t r);
int lq_qlora_backward_noalloc(const lq_qweight* w, const uint16_t* X, const uint16_t* G, int64_t M,
                              const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                              const float* t_saved, uint16_t* grad_X, float* dA, float* dB, void* stream);

/* ---- checks and the LQ_DEBUG build ---------------------------------------- */

/*
 * Host check of a codebook weight's layout and tables ([LowRA] section 3:
 * per-output-channel precision and thresholds), on HOST arrays:
 *   row_bits   [N] uint8, each in {1, 2, 3, 4}
 *   row_offset [N + 1] int64, row_offset[0] = 0 and
 *              row_offset[i+1] - row_offset[i] = K * row_bits[i] / 8
 *   thresholds [N, 15] float32 or NULL: the first 2^b - 1 of row i finite and
 *              strictly increasing
 * Returns LQ_OK, LQ_ERR_SHAPE (N <= 0, K <= 0, K % 64 != 0) or LQ_ERR_ARG
 * (a null array or the first violation found). Pure host function.
 */
int lq_check_codebook_tables(int64_t N, int64_t K, const uint8_t* row_bits, const int64_t* row_offset,
                             const float* thresholds);

/* 1 in the LQ_DEBUG build (liblq_debug.so), 0 in the release build. */
int lq_debug_build(void);

/* Bits of the debug build's device flag word. */
#define LQ_DBG_NONFINITE 1u   /* a quantizer read a NaN or infinite weight */
#define LQ_DBG_THRESHOLDS 2u  /* a codebook row's thresholds are not strictly increasing */
#define LQ_DBG_ROW_BITS 4u    /* a codebook row width outside 1..4 (clamped into it) */

/*
 * Debug build only: the flag word of the current device (LQ_DBG_* bits set by
 * the quantizers since it was last cleared), read after synchronising the
 * device; cleared to 0 afterwards if `clear` is non-zero. The debug build
 * also checks, before launching, the row layout of codebook weights passed to
 * lq_quantize_codebook, lq_dequant, lq_qlora_forward, lq_dequant_gemm,
 * lq_dequant_gemm_t and lq_qlora_backward (it copies row_bits and row_offset
 * to the host on the caller's stream and synchronises it; LQ_ERR_ARG on a
 * violation), and asserts its launch-shape assumptions on the host
 * (LQ_ERR_LAUNCH if one fails, with a message on stderr).
 *   flags  host uint32, written
 * Errors: LQ_ERR_ARG (flags NULL), LQ_ERR_UNSUPPORTED (release build),
 * LQ_ERR_LAUNCH (runtime error).
 */
int lq_debug_flags(uint32_t* flags, int clear);

#ifdef __cplusplus
}
#endif

#endif /* LQ_H */
