// The C ABI of include/lq.h: argument validation, workspace carving and
// kernel dispatch. No device memory is allocated here; every launch goes on
// the caller's stream.
#include <cmath>
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lq_internal.h"

namespace {

using namespace lq;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int32_t d) { return d == LQ_F32 || d == LQ_BF16 || d == LQ_F16; }

int launch_status(hipError_t e) { return e == hipSuccess ? LQ_OK : LQ_ERR_LAUNCH; }

// Alignment of a device pointer (a null pointer passes; nullness is checked
// separately). Bulk tensors are read and written with 16-byte vector
// accesses; per-element arrays need their natural alignment.
constexpr uintptr_t kVec = 16;
bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
// W of the NF4 quantizer and the profiling pass: four elements per access
uintptr_t w_align(int32_t dtype) { return dtype == LQ_F32 ? 16 : 8; }

// Validate a weight descriptor and turn it into the kernels' view.
int check_qweight(const lq_qweight* w, QWeight* out) {
  if (!w) return LQ_ERR_ARG;
  if (w->format != LQ_FMT_NF4 && w->format != LQ_FMT_CODEBOOK) return LQ_ERR_ARG;
  if (w->blocksize != 64) return LQ_ERR_UNSUPPORTED;
  if (w->N <= 0 || w->K <= 0 || w->K % 64 != 0) return LQ_ERR_SHAPE;
  if (!w->codes) return LQ_ERR_ARG;
  if (!w->absmax) {
    if (!w->absmax_q || !w->dq_scale || !w->dq_mean) return LQ_ERR_ARG;
    if (w->dq_blocksize != 256) return LQ_ERR_UNSUPPORTED;
  }
  if (w->format == LQ_FMT_CODEBOOK && (!w->row_bits || !w->row_offset || !w->levels)) return LQ_ERR_ARG;
  if (!al(w->codes, kVec) || !al(w->absmax, 4) || !al(w->absmax_q, kVec) || !al(w->dq_scale, 4) ||
      !al(w->dq_mean, 4) || !al(w->row_offset, 8) || !al(w->levels, 4))
    return LQ_ERR_ARG;
  out->format = w->format;
  out->N = w->N;
  out->K = w->K;
  out->codes = w->codes;
  out->qc.absmax = w->absmax;
  out->qc.absmax_q = w->absmax ? nullptr : w->absmax_q;
  out->qc.dq_scale = w->absmax ? nullptr : w->dq_scale;
  out->qc.dq_mean = w->absmax ? nullptr : w->dq_mean;
  out->row_bits = w->row_bits;
  out->row_offset = w->row_offset;
  out->levels = w->levels;
  return LQ_OK;
}

// Forward path choice: the GEMV kernel for decode-sized M, else the MFMA
// GEMM. LQ_FORCE_PATH=gemm forces the GEMM at any M (for tests).
bool use_gemv(const QWeight& w, int64_t M) {
  if (M > 16 || !gemv_supported(w)) return false;
  const char* f = std::getenv("LQ_FORCE_PATH");
  if (f && std::strcmp(f, "gemm") == 0) return false;
  return true;
}

// Carves a caller workspace into aligned pieces; ok() is false if the pieces
// ran past its size (the entry points size the workspace first, so this is a
// bounds assert on that arithmetic).
struct Carver {
  char* base;
  size_t cap;
  size_t used = 0;
  Carver(void* p, size_t bytes) : base((char*)p), cap(bytes) {}
  template <class T> T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base + used);
    used += align_up(count * sizeof(T));
    return p;
  }
  bool ok() const { return used <= cap; }
};

// Row layout of a codebook weight (host arrays): widths in 1..4, offsets the
// prefix sums of K*b/8; thresholds (optional) finite and strictly increasing.
int check_codebook_host(int64_t N, int64_t K, const uint8_t* bits, const int64_t* off, const float* T) {
  if (off[0] != 0) return LQ_ERR_ARG;
  for (int64_t i = 0; i < N; ++i) {
    const int b = bits[i];
    if (b < 1 || b > 4) return LQ_ERR_ARG;
    if (off[i + 1] - off[i] != K * b / 8) return LQ_ERR_ARG;
    if (T) {
      const float* t = T + i * 15;
      for (int k = 0; k < (1 << b) - 1; ++k) {
        if (!std::isfinite(t[k])) return LQ_ERR_ARG;
        if (k > 0 && !(t[k] > t[k - 1])) return LQ_ERR_ARG;
      }
    }
  }
  return LQ_OK;
}

// Debug build: copy a codebook weight's row_bits and row_offset to the host
// (in order on the caller's stream) and check the layout before launching.
int debug_check_rows(int64_t N, int64_t K, const uint8_t* bits_d, const int64_t* off_d, hipStream_t s) {
#ifdef LQ_DEBUG
  std::vector<uint8_t> bits((size_t)N);
  std::vector<int64_t> off((size_t)N + 1);
  if (hipMemcpyAsync(bits.data(), bits_d, (size_t)N, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(off.data(), off_d, ((size_t)N + 1) * sizeof(int64_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return LQ_ERR_LAUNCH;
  return check_codebook_host(N, K, bits.data(), off.data(), nullptr);
#else
  (void)N; (void)K; (void)bits_d; (void)off_d; (void)s;
  return LQ_OK;
#endif
}
int debug_check_weight(const QWeight& q, hipStream_t s) {
  return q.format == LQ_FMT_CODEBOOK ? debug_check_rows(q.N, q.K, q.row_bits, q.row_offset, s) : LQ_OK;
}

// Column parts of t = X A^T in the forward: only for the NF4 GEMV, which adds
// them while staging t (the GEMM takes t whole: summing parts in its LoRA
// step cost it registers it does not have).
int forward_t_parts(const QWeight& w, int64_t M) {
  return (use_gemv(w, M) && w.format == LQ_FMT_NF4) ? row_skinny_parts(M, w.K) : 1;
}

// t (as column-part partial sums), GEMM workspace
size_t forward_ws(const QWeight& w, int64_t M, int32_t r) {
  return align_up((size_t)forward_t_parts(w, M) * M * r * sizeof(float)) +
         (use_gemv(w, M) ? 0 : align_up(gemm_ws_bytes(w, M, r, true)));
}

// u, recomputed t, B^T, split t and u, partial sums of dB and of dA, GEMM
// workspace. (u and t are formed whole here: split into column parts, the
// row-form product got 4 us faster at q_proj but the column form that adds
// the parts 2.5 us slower.)
size_t backward_ws(const QWeight& w, int64_t M, int32_t r) {
  return 2 * align_up((size_t)M * r * sizeof(float)) +
         (r > 16 ? align_up((size_t)w.N * r * sizeof(uint16_t)) : 0) +
         align_up(col_skinny_ws_floats(M, w.N, r) * sizeof(float)) +
         align_up(col_skinny_ws_floats(M, w.K, r) * sizeof(float)) + align_up(gemm_ws_bytes(w, M, r, false));
}

// Arguments of the backward entry points, validated before anything runs.
int check_backward(const lq_qweight* w, QWeight* q, const uint16_t* X, const uint16_t* G, int64_t M,
                   const uint16_t* A, const uint16_t* B, int32_t r, const float* t_saved, const uint16_t* grad_X,
                   const float* dA, const float* dB) {
  const int st = check_qweight(w, q);
  if (st != LQ_OK) return st;
  if (!G || !A || !B) return LQ_ERR_ARG;
  if ((dA || !t_saved) && !X) return LQ_ERR_ARG;
  if (!al(X, kVec) || !al(G, kVec) || !al(A, kVec) || !al(B, kVec) || !al(t_saved, 4) || !al(grad_X, kVec) ||
      !al(dA, 4) || !al(dB, 4))
    return LQ_ERR_ARG;
  if (M <= 0 || r < 1 || r > 128 || q->N % 8 != 0) return LQ_ERR_SHAPE;
  return LQ_OK;
}

// The backward's launches over a workspace of at least backward_ws bytes
// (whose contents on entry do not matter: every piece is written before it
// is read).
int run_backward(const QWeight& q, const uint16_t* X, const uint16_t* G, int64_t M, const uint16_t* A,
                 const uint16_t* B, int32_t r, float alpha, const float* t_saved, uint16_t* grad_X, float* dA,
                 float* dB, void* workspace, size_t ws_bytes, hipStream_t s) {
  Carver cv(workspace, ws_bytes);
  float* u = cv.take<float>((size_t)M * r);
  float* t_ws = cv.take<float>((size_t)M * r);
  uint16_t* Bt = r > 16 ? cv.take<uint16_t>((size_t)q.N * r) : nullptr;
  float* part_b = cv.take<float>(col_skinny_ws_floats(M, q.N, r));
  float* part_a = cv.take<float>(col_skinny_ws_floats(M, q.K, r));
  uint16_t* gws = cv.take<uint16_t>(gemm_ws_bytes(q, M, r, false) / sizeof(uint16_t));
  if (!cv.ok()) return LQ_ERR_WORKSPACE;
  int st = debug_check_weight(q, s);
  if (st != LQ_OK) return st;
  const float scale = alpha / (float)r;
  hipError_t e = hipSuccess;
  const float* t = t_saved;
  if (!t) {
    e = launch_row_skinny(X, M, q.K, A, r, t_ws, s);
    if (e != hipSuccess) return LQ_ERR_LAUNCH;
    t = t_ws;
  }
  // u = G B: B read as given ([N, r]) up to r = 16, else transposed first
  if (r <= 16) {
    e = launch_row_skinny_rt(G, M, q.N, B, r, u, s);
  } else {
    e = launch_transpose_u16(B, q.N, r, Bt, s);
    if (e == hipSuccess) e = launch_row_skinny(G, M, q.N, Bt, r, u, s);
  }
  if (e != hipSuccess) return LQ_ERR_LAUNCH;
  // partial sums of dB = s G^T t and dA = s u^T X in one launch
  SplitJobDesc job_b, job_a;
  const ColSkinnyReq req_b{t, G, q.N, scale, dB, true, part_b};
  const ColSkinnyReq req_a{u, X, q.K, scale, dA, false, part_a};
  e = launch_col_skinny(dB ? &req_b : nullptr, dA ? &req_a : nullptr, M, r, &job_b, &job_a, s);
  if (e != hipSuccess) return LQ_ERR_LAUNCH;
  // grad_X; its workgroups also finish dB and dA from the partial sums
  if (grad_X) return launch_status(launch_gemm_bwd(q, G, M, u, A, r, scale, grad_X, gws, s, &job_b, &job_a));
  return launch_status(launch_reduce_splits2(job_b, job_a, s));
}

}  // namespace

extern "C" {

const char* lq_status_string(int status) {
  switch (status) {
    case LQ_OK: return "ok";
    case LQ_ERR_ARG: return "invalid argument (null pointer, misaligned pointer or bad enum value)";
    case LQ_ERR_SHAPE: return "invalid shape (sizes must be positive, K % 64 == 0, r in [1, 128])";
    case LQ_ERR_UNSUPPORTED: return "unsupported option (blocksize, double-quant blocksize or dtype)";
    case LQ_ERR_WORKSPACE: return "workspace missing or too small";
    case LQ_ERR_LAUNCH: return "HIP runtime error at kernel launch";
    default: return "unknown status";
  }
}

int lq_version(void) { return 100; }

int lq_nf4_table(float* levels, float* thresholds) {
  const Tables& t = tables();
  if (levels) std::memcpy(levels, t.levels, sizeof(t.levels));
  if (thresholds) std::memcpy(thresholds, t.thresholds, sizeof(t.thresholds));
  return LQ_OK;
}

int lq_sizes(int64_t N, int64_t K, int32_t bits, lq_sizes_t* out) {
  if (!out || bits < 1 || bits > 4) return LQ_ERR_ARG;
  if (N <= 0 || K <= 0 || K % 64 != 0) return LQ_ERR_SHAPE;
  out->n = N * K;
  out->n_blocks = out->n / 64;
  out->n_dq_blocks = (out->n_blocks + 255) / 256;
  out->code_bytes = out->n * bits / 8;
  out->dq_const_bytes = out->n_blocks + 4 * out->n_dq_blocks + 4;
  out->fp32_const_bytes = 4 * out->n_blocks;
  out->const_bits_per_param_dq = 8.0 / 64.0 + 32.0 / (64.0 * 256.0);
  out->const_bits_per_param_fp32 = 32.0 / 64.0;
  return LQ_OK;
}

int lq_quantize_nf4(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize,
                    uint8_t* codes, float* absmax, void* stream) {
  if (!W || !codes || !absmax || !valid_dtype(dtype)) return LQ_ERR_ARG;
  if (!al(W, w_align(dtype)) || !al(codes, 8) || !al(absmax, 4)) return LQ_ERR_ARG;
  if (N <= 0 || K <= 0 || K % 64 != 0) return LQ_ERR_SHAPE;
  if (blocksize != 64) return LQ_ERR_UNSUPPORTED;
  return launch_status(launch_quantize_nf4(W, dtype, N * K / 64, codes, absmax, (hipStream_t)stream));
}

size_t lq_profile_workspace(int64_t N, int64_t K, int32_t blocksize) {
  if (N <= 0 || K <= 0 || K % 64 != 0 || blocksize != 64) return 0;
  return align_up(profile_ws_doubles(N * K / 64) * sizeof(double));
}

int lq_profile_nf4(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize, double tau,
                   double* stats, void* workspace, size_t ws_bytes, void* stream) {
  if (!W || !stats || !valid_dtype(dtype)) return LQ_ERR_ARG;
  if (!al(W, w_align(dtype)) || !al(stats, 8) || !al(workspace, kVec)) return LQ_ERR_ARG;
  if (N <= 0 || K <= 0 || K % 64 != 0) return LQ_ERR_SHAPE;
  if (blocksize != 64) return LQ_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < lq_profile_workspace(N, K, blocksize)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_profile_nf4(W, dtype, N * K / 64, tau, stats, (double*)workspace,
                                          (hipStream_t)stream));
}

size_t lq_double_quant_workspace(int64_t n_blocks, int32_t dq_blocksize) {
  if (n_blocks <= 0 || dq_blocksize != 256) return 0;
  return align_up(double_quant_ws_doubles(n_blocks) * sizeof(double));
}

int lq_double_quant(const float* absmax, int64_t n_blocks, int32_t dq_blocksize,
                    uint8_t* absmax_q, float* dq_scale, float* dq_mean, void* workspace,
                    size_t ws_bytes, void* stream) {
  if (!absmax || !absmax_q || !dq_scale || !dq_mean) return LQ_ERR_ARG;
  if (!al(absmax, 4) || !al(dq_scale, 4) || !al(dq_mean, 4) || !al(workspace, kVec)) return LQ_ERR_ARG;
  if (n_blocks <= 0) return LQ_ERR_SHAPE;
  if (dq_blocksize != 256) return LQ_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < lq_double_quant_workspace(n_blocks, dq_blocksize)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_double_quant(absmax, n_blocks, absmax_q, dq_scale, dq_mean,
                                           (double*)workspace, (hipStream_t)stream));
}

int lq_double_quant_dequant(const float* absmax, int64_t n_blocks, int32_t dq_blocksize,
                            uint8_t* absmax_q, float* dq_scale, float* dq_mean, const uint8_t* codes,
                            uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!absmax || !absmax_q || !dq_scale || !dq_mean || !codes || !out) return LQ_ERR_ARG;
  if (!al(absmax, 4) || !al(dq_scale, 4) || !al(dq_mean, 4) || !al(codes, kVec) || !al(out, kVec) ||
      !al(workspace, kVec))
    return LQ_ERR_ARG;
  if (n_blocks <= 0) return LQ_ERR_SHAPE;
  if (dq_blocksize != 256) return LQ_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < lq_double_quant_workspace(n_blocks, dq_blocksize)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_double_quant_dequant(absmax, n_blocks, absmax_q, dq_scale, dq_mean, codes, out,
                                                   (double*)workspace, (hipStream_t)stream));
}

int lq_dequant(const lq_qweight* w, uint16_t* out, void* stream) {
  QWeight q;
  const int st = check_qweight(w, &q);
  if (st != LQ_OK) return st;
  if (!out || !al(out, kVec)) return LQ_ERR_ARG;
  const int dc = debug_check_weight(q, (hipStream_t)stream);
  if (dc != LQ_OK) return dc;
  return launch_status(launch_dequant(q, out, (hipStream_t)stream));
}

size_t lq_forward_workspace(const lq_qweight* w, int64_t M, int32_t r) {
  QWeight q;
  if (check_qweight(w, &q) != LQ_OK || M <= 0 || r < 1 || r > 128) return 0;
  return forward_ws(q, M, r);
}

int lq_qlora_forward(const lq_qweight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha, void* H, int32_t h_dtype,
                     float* t_save, void* workspace, size_t ws_bytes, void* stream) {
  QWeight q;
  int st = check_qweight(w, &q);
  if (st != LQ_OK) return st;
  if (!X || !A || !B || !H) return LQ_ERR_ARG;
  if (!al(X, kVec) || !al(A, kVec) || !al(B, kVec) || !al(H, h_dtype == LQ_F32 ? 4 : kVec) || !al(t_save, 4) ||
      !al(workspace, kVec))
    return LQ_ERR_ARG;
  if (M <= 0 || r < 1 || r > 128) return LQ_ERR_SHAPE;
  if (h_dtype != LQ_BF16 && h_dtype != LQ_F32) return LQ_ERR_UNSUPPORTED;
  const size_t need = forward_ws(q, M, r);
  if (!workspace || ws_bytes < need) return LQ_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Carver cv(workspace, ws_bytes);
  const bool gemv = use_gemv(q, M);
  const int parts = forward_t_parts(q, M);
  float* t_ws = cv.take<float>((size_t)parts * M * r);
  uint16_t* gws = gemv ? nullptr : cv.take<uint16_t>(gemm_ws_bytes(q, M, r, true) / sizeof(uint16_t));
  if (!cv.ok()) return LQ_ERR_WORKSPACE;
  if ((st = debug_check_weight(q, s)) != LQ_OK) return st;
  float* t = t_save ? t_save : t_ws;
  const float scale = alpha / (float)r;
  // decode sizes with a small NF4 weight and r <= 32: the GEMV forms t itself
  if (gemv && gemv_forms_t(q, M, r))
    return launch_status(launch_gemv_fwd(q, X, M, nullptr, B, r, scale, H, h_dtype, s, A, t));
  // t = X A^T; for the GEMV split into column parts, which the GEMV adds
  // (storing t) while staging it
  const float* tin = parts > 1 ? t_ws : t;
  hipError_t e = launch_row_skinny(X, M, q.K, A, r, parts > 1 ? t_ws : t, s, parts);
  if (e != hipSuccess) return LQ_ERR_LAUNCH;
  if (gemv) e = launch_gemv_fwd(q, X, M, tin, B, r, scale, H, h_dtype, s, nullptr, t_save, parts);
  else e = launch_gemm_fwd(q, X, M, tin, B, r, scale, H, h_dtype, gws, s);
  return launch_status(e);
}

size_t lq_lora_down_workspace(int64_t, int64_t, int32_t) { return 0; }

int lq_lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int32_t r, float* t,
                 void* workspace, size_t ws_bytes, void* stream) {
  if (!X || !A || !t) return LQ_ERR_ARG;
  if (!al(X, kVec) || !al(A, kVec) || !al(t, 4)) return LQ_ERR_ARG;
  if (M <= 0 || K <= 0 || K % 8 != 0 || r < 1 || r > 128) return LQ_ERR_SHAPE;
  (void)workspace;
  (void)ws_bytes;
  return launch_status(launch_row_skinny(X, M, K, A, r, t, (hipStream_t)stream));
}

size_t lq_dequant_gemm_workspace(const lq_qweight* w, int64_t M, int32_t r) {
  QWeight q;
  if (check_qweight(w, &q) != LQ_OK || M <= 0 || r < 1 || r > 128) return 0;
  if (use_gemv(q, M)) return 0;   // the GEMV kernel reads t and B directly
  return align_up(gemm_ws_bytes(q, M, r, true));
}

int lq_dequant_gemm(const lq_qweight* w, const uint16_t* X, int64_t M, const float* t,
                    const uint16_t* B, int32_t r, float alpha, void* H, int32_t h_dtype,
                    void* workspace, size_t ws_bytes, void* stream) {
  QWeight q;
  const int st = check_qweight(w, &q);
  if (st != LQ_OK) return st;
  if (!X || !t || !B || !H) return LQ_ERR_ARG;
  if (!al(X, kVec) || !al(t, 4) || !al(B, kVec) || !al(H, h_dtype == LQ_F32 ? 4 : kVec) || !al(workspace, kVec))
    return LQ_ERR_ARG;
  if (M <= 0 || r < 1 || r > 128) return LQ_ERR_SHAPE;
  if (h_dtype != LQ_BF16 && h_dtype != LQ_F32) return LQ_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const float scale = alpha / (float)r;
  const int dc = debug_check_weight(q, s);
  if (dc != LQ_OK) return dc;
  if (use_gemv(q, M)) return launch_status(launch_gemv_fwd(q, X, M, t, B, r, scale, H, h_dtype, s));
  const size_t need = gemm_ws_bytes(q, M, r, true);
  if (need && (!workspace || ws_bytes < need)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_gemm_fwd(q, X, M, t, B, r, scale, H, h_dtype, (uint16_t*)workspace, s));
}

size_t lq_dequant_gemm_t_workspace(const lq_qweight* w, int64_t M, int32_t r) {
  QWeight q;
  if (check_qweight(w, &q) != LQ_OK || M <= 0 || r < 1 || r > 128) return 0;
  return align_up(gemm_ws_bytes(q, M, r, false));
}

int lq_dequant_gemm_t(const lq_qweight* w, const uint16_t* G, int64_t M, const float* u,
                      const uint16_t* A, int32_t r, float alpha, uint16_t* grad_X,
                      void* workspace, size_t ws_bytes, void* stream) {
  QWeight q;
  const int st = check_qweight(w, &q);
  if (st != LQ_OK) return st;
  if (!G || !u || !A || !grad_X) return LQ_ERR_ARG;
  if (!al(G, kVec) || !al(u, 4) || !al(A, kVec) || !al(grad_X, kVec) || !al(workspace, kVec)) return LQ_ERR_ARG;
  if (M <= 0 || r < 1 || r > 128 || q.N % 8 != 0) return LQ_ERR_SHAPE;
  const size_t need = gemm_ws_bytes(q, M, r, false);
  if (need && (!workspace || ws_bytes < need)) return LQ_ERR_WORKSPACE;
  const int dc = debug_check_weight(q, (hipStream_t)stream);
  if (dc != LQ_OK) return dc;
  return launch_status(launch_gemm_bwd(q, G, M, u, A, r, alpha / (float)r, grad_X, (uint16_t*)workspace,
                                       (hipStream_t)stream));
}

size_t lq_backward_workspace(const lq_qweight* w, int64_t M, int32_t r) {
  QWeight q;
  if (check_qweight(w, &q) != LQ_OK || M <= 0 || r < 1 || r > 128) return 0;
  return backward_ws(q, M, r);
}

int lq_qlora_backward(const lq_qweight* w, const uint16_t* X, const uint16_t* G, int64_t M,
                      const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                      const float* t_saved, uint16_t* grad_X, float* dA, float* dB,
                      void* workspace, size_t ws_bytes, void* stream) {
  QWeight q;
  const int st = check_backward(w, &q, X, G, M, A, B, r, t_saved, grad_X, dA, dB);
  if (st != LQ_OK) return st;
  if (!al(workspace, kVec)) return LQ_ERR_ARG;
  if (!workspace || ws_bytes < backward_ws(q, M, r)) return LQ_ERR_WORKSPACE;
  return run_backward(q, X, G, M, A, B, r, alpha, t_saved, grad_X, dA, dB, workspace, ws_bytes,
                      (hipStream_t)stream);
}

size_t lq_qlora_backward_noalloc_bytes(const lq_qweight* w, int64_t M, int32_t r) {
  return lq_backward_workspace(w, M, r);
}

int lq_qlora_backward_noalloc(const lq_qweight* w, const uint16_t* X, const uint16_t* G, int64_t M,
                              const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                              const float* t_saved, uint16_t* grad_X, float* dA, float* dB, void* stream) {
  QWeight q;
  const int st = check_backward(w, &q, X, G, M, A, B, r, t_saved, grad_X, dA, dB);
  if (st != LQ_OK) return st;
  if (backward_ws(q, M, r) > (size_t)LQ_NOALLOC_SCRATCH_BYTES) return LQ_ERR_WORKSPACE;
  void* scratch = nullptr;   // this device's copy of the library's scratch array
  if (noalloc_scratch(&scratch) != hipSuccess) return LQ_ERR_LAUNCH;
  return run_backward(q, X, G, M, A, B, r, alpha, t_saved, grad_X, dA, dB, scratch,
                      (size_t)LQ_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}

int lq_quantize_codebook(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize,
                         const uint8_t* row_bits, const int64_t* row_offset,
                         const float* thresholds, uint8_t* codes, float* absmax, void* stream) {
  if (!W || !row_bits || !row_offset || !thresholds || !codes || !absmax || !valid_dtype(dtype))
    return LQ_ERR_ARG;
  if (!al(W, dtype == LQ_F32 ? 4 : 2) || !al(row_offset, 8) || !al(thresholds, 4) || !al(codes, 4) ||
      !al(absmax, 4))
    return LQ_ERR_ARG;
  if (N <= 0 || K <= 0 || K % 64 != 0) return LQ_ERR_SHAPE;
  if (blocksize != 64) return LQ_ERR_UNSUPPORTED;
  const int dc = debug_check_rows(N, K, row_bits, row_offset, (hipStream_t)stream);
  if (dc != LQ_OK) return dc;
  return launch_status(launch_quantize_codebook(W, dtype, N, K, row_bits, row_offset, thresholds,
                                                codes, absmax, (hipStream_t)stream));
}

int lq_lloyd_codebooks(const void* W, int32_t dtype, int64_t N, int64_t K, int32_t blocksize,
                       const uint8_t* row_bits, int32_t max_iters, float* levels,
                       float* thresholds, int32_t* iterations, void* stream) {
  if (!W || !row_bits || !levels || !thresholds || !valid_dtype(dtype)) return LQ_ERR_ARG;
  if (!al(W, dtype == LQ_F32 ? 4 : 2) || !al(levels, 4) || !al(thresholds, 4) || !al(iterations, 4))
    return LQ_ERR_ARG;
  if (max_iters < 1 || max_iters > LQ_LLOYD_MAX_ITERS_LIMIT) return LQ_ERR_ARG;
  if (N <= 0 || K <= 0 || K % 64 != 0 || N > INT32_MAX) return LQ_ERR_SHAPE;
  if (blocksize != 64 || K > LQ_LLOYD_MAX_K) return LQ_ERR_UNSUPPORTED;
  return launch_status(launch_lloyd(W, dtype, N, K, row_bits, max_iters, levels, thresholds,
                                    iterations, (hipStream_t)stream));
}

int lq_lowrank_sub(const float* W, int64_t N, int64_t K, const float* B, const float* A, int32_t r,
                   float* out, void* stream) {
  if (!W || !out || (r > 0 && (!B || !A))) return LQ_ERR_ARG;
  if (!al(W, kVec) || !al(out, kVec) || !al(A, kVec) || !al(B, 4)) return LQ_ERR_ARG;
  if (N <= 0 || K <= 0 || K % 4 != 0 || r < 0 || r > 128) return LQ_ERR_SHAPE;
  return launch_status(launch_lowrank_sub(W, N, K, B, A, r, out, (hipStream_t)stream));
}

int lq_residual(const float* W, const uint16_t* Wd, int64_t n, float* R, void* stream) {
  if (!W || !Wd || !R) return LQ_ERR_ARG;
  if (!al(W, kVec) || !al(Wd, 8) || !al(R, kVec)) return LQ_ERR_ARG;
  if (n <= 0 || n % 4 != 0) return LQ_ERR_SHAPE;
  return launch_status(launch_residual(W, Wd, n, R, (hipStream_t)stream));
}

static int check_svd_shape(int64_t N, int64_t K, int32_t r, int32_t l, int32_t power_iters) {
  if (N <= 0 || K <= 0 || K % 4 != 0 || r < 1 || l < r || l % 2 != 0 || l > N || l > K) return LQ_ERR_SHAPE;
  if (l > lowrank_max_l()) return LQ_ERR_UNSUPPORTED;
  if (power_iters < 0 || power_iters > 1000) return LQ_ERR_ARG;
  return LQ_OK;
}

size_t lq_svd_lowrank_workspace(int64_t N, int64_t K, int32_t r, int32_t l) {
  if (check_svd_shape(N, K, r, l, 0) != LQ_OK) return 0;
  return align_up(svd_ws_bytes(N, K, l, r));
}

int lq_svd_lowrank(const float* R, int64_t N, int64_t K, int32_t r, int32_t l, int32_t power_iters,
                   const float* omega, float* B, float* A, float* sigma, void* workspace, size_t ws_bytes,
                   void* stream) {
  if (!R || !omega || !B || !A || !sigma) return LQ_ERR_ARG;
  if (!al(R, kVec) || !al(omega, kVec) || !al(B, kVec) || !al(A, kVec) || !al(sigma, 4) || !al(workspace, kVec))
    return LQ_ERR_ARG;
  const int st = check_svd_shape(N, K, r, l, power_iters);
  if (st != LQ_OK) return st;
  if (!workspace || ws_bytes < svd_ws_bytes(N, K, l, r)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_svd_lowrank(R, N, K, r, l, power_iters, omega, B, A, sigma, workspace,
                                          (hipStream_t)stream));
}

size_t lq_loftq_workspace(int64_t N, int64_t K, int32_t r, int32_t l, int32_t double_quant) {
  if (K % 64 != 0 || check_svd_shape(N, K, r, l, 0) != LQ_OK) return 0;
  return align_up(loftq_ws_bytes(N, K, r, l, double_quant != 0));
}

int lq_loftq_init(const float* W, int64_t N, int64_t K, int32_t blocksize, int32_t double_quant, int32_t r,
                  int32_t l, int32_t steps, int32_t power_iters, const float* omega, uint8_t* codes,
                  float* absmax, uint8_t* absmax_q, float* dq_scale, float* dq_mean, float* B, float* A,
                  float* sigma, double* objectives, void* workspace, size_t ws_bytes, void* stream) {
  const bool dq = double_quant != 0;
  if (!W || !omega || !codes || !absmax || !B || !A || !sigma) return LQ_ERR_ARG;
  if (dq && (!absmax_q || !dq_scale || !dq_mean)) return LQ_ERR_ARG;
  if (!al(W, kVec) || !al(omega, kVec) || !al(codes, kVec) || !al(absmax, 4) || !al(absmax_q, kVec) ||
      !al(dq_scale, 4) || !al(dq_mean, 4) || !al(B, kVec) || !al(A, kVec) || !al(sigma, 4) || !al(objectives, 8) ||
      !al(workspace, kVec))
    return LQ_ERR_ARG;
  if (steps < 1 || steps > 100) return LQ_ERR_ARG;
  if (K % 64 != 0) return LQ_ERR_SHAPE;
  const int st = check_svd_shape(N, K, r, l, power_iters);
  if (st != LQ_OK) return st;
  if (blocksize != 64) return LQ_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < loftq_ws_bytes(N, K, r, l, dq)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_loftq(W, N, K, dq, r, l, steps, power_iters, omega, codes, absmax, absmax_q,
                                    dq_scale, dq_mean, B, A, sigma, objectives, workspace, (hipStream_t)stream));
}

static int check_loraquant_shape(int64_t N, int64_t K, int32_t r) {
  if (N <= 0 || K <= 0 || N % 64 != 0 || K % 64 != 0 || r < 1) return LQ_ERR_SHAPE;
  if (r > LQ_LORAQUANT_MAX_R || N > LQ_LLOYD_MAX_K || K > LQ_LLOYD_MAX_K) return LQ_ERR_UNSUPPORTED;
  return LQ_OK;
}

size_t lq_loraquant_workspace(int64_t N, int64_t K, int32_t r) {
  if (check_loraquant_shape(N, K, r) != LQ_OK) return 0;
  return align_up(loraquant_ws_bytes(N, K, r));
}

int lq_loraquant(const float* B, const float* A, int64_t N, int64_t K, int32_t r, double rho, int32_t h,
                 int32_t bits_hi, int32_t bits_lo, uint8_t* codes_a, float* absmax_a, uint8_t* codes_b,
                 float* absmax_b, uint8_t* row_bits, int64_t* offsets_a, int64_t* offsets_b, float* levels_a,
                 float* thresholds_a, float* levels_b, float* thresholds_b, float* sigma, int32_t* h_out, float* Ap,
                 float* Bpt, void* workspace, size_t ws_bytes, void* stream) {
  if (!B || !A || !codes_a || !absmax_a || !codes_b || !absmax_b || !row_bits || !offsets_a || !offsets_b ||
      !levels_a || !thresholds_a || !levels_b || !thresholds_b || !sigma || !h_out)
    return LQ_ERR_ARG;
  if (bits_hi < 1 || bits_hi > 4 || bits_lo < 1 || bits_lo > 4 || h > r) return LQ_ERR_ARG;
  if (!al(B, kVec) || !al(A, kVec) || !al(codes_a, kVec) || !al(codes_b, kVec) || !al(absmax_a, 4) ||
      !al(absmax_b, 4) || !al(offsets_a, 8) || !al(offsets_b, 8) || !al(levels_a, 4) || !al(levels_b, 4) ||
      !al(thresholds_a, 4) || !al(thresholds_b, 4) || !al(sigma, 4) || !al(h_out, 4) || !al(Ap, kVec) ||
      !al(Bpt, kVec) || !al(workspace, kVec))
    return LQ_ERR_ARG;
  const int st = check_loraquant_shape(N, K, r);
  if (st != LQ_OK) return st;
  if (!workspace || ws_bytes < loraquant_ws_bytes(N, K, r)) return LQ_ERR_WORKSPACE;
  return launch_status(launch_loraquant(B, A, N, K, r, rho, h, bits_hi, bits_lo, codes_a, absmax_a, codes_b,
                                        absmax_b, row_bits, offsets_a, offsets_b, levels_a, thresholds_a, levels_b,
                                        thresholds_b, sigma, h_out, Ap, Bpt, workspace, (hipStream_t)stream));
}

size_t lq_loraquant_dequant_workspace(int64_t N, int64_t K, int32_t r) {
  if (check_loraquant_shape(N, K, r) != LQ_OK) return 0;
  return align_up((size_t)N * r * sizeof(uint16_t));
}

int lq_loraquant_dequant(const uint8_t* codes_a, const float* absmax_a, const uint8_t* codes_b,
                         const float* absmax_b, const uint8_t* row_bits, const int64_t* offsets_a,
                         const int64_t* offsets_b, const float* levels_a, const float* levels_b, int64_t N,
                         int64_t K, int32_t r, uint16_t* A_bf16, uint16_t* B_bf16, void* workspace, size_t ws_bytes,
                         void* stream) {
  if (!codes_a || !absmax_a || !codes_b || !absmax_b || !row_bits || !offsets_a || !offsets_b || !levels_a ||
      !levels_b || !A_bf16 || !B_bf16)
    return LQ_ERR_ARG;
  if (!al(codes_a, kVec) || !al(codes_b, kVec) || !al(absmax_a, 4) || !al(absmax_b, 4) || !al(offsets_a, 8) ||
      !al(offsets_b, 8) || !al(levels_a, 4) || !al(levels_b, 4) || !al(A_bf16, kVec) || !al(B_bf16, kVec) ||
      !al(workspace, kVec))
    return LQ_ERR_ARG;
  const int st = check_loraquant_shape(N, K, r);
  if (st != LQ_OK) return st;
  if (!workspace || ws_bytes < (size_t)N * r * sizeof(uint16_t)) return LQ_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  QWeight qa{};
  qa.format = LQ_FMT_CODEBOOK;
  qa.N = r;
  qa.K = K;
  qa.codes = codes_a;
  qa.qc = QConst{absmax_a, nullptr, nullptr, nullptr};
  qa.row_bits = row_bits;
  qa.row_offset = offsets_a;
  qa.levels = levels_a;
  QWeight qb = qa;
  qb.K = N;
  qb.codes = codes_b;
  qb.qc = QConst{absmax_b, nullptr, nullptr, nullptr};
  qb.row_offset = offsets_b;
  qb.levels = levels_b;
  hipError_t e = launch_dequant(qa, A_bf16, s);
  if (e != hipSuccess) return LQ_ERR_LAUNCH;
  uint16_t* bt = (uint16_t*)workspace;   // B'^T [r, N]
  e = launch_dequant(qb, bt, s);
  if (e != hipSuccess) return LQ_ERR_LAUNCH;
  return launch_status(launch_transpose_u16(bt, r, (int)N, B_bf16, s));
}

int lq_check_codebook_tables(int64_t N, int64_t K, const uint8_t* row_bits, const int64_t* row_offset,
                             const float* thresholds) {
  if (N <= 0 || K <= 0 || K % 64 != 0) return LQ_ERR_SHAPE;
  if (!row_bits || !row_offset) return LQ_ERR_ARG;
  return check_codebook_host(N, K, row_bits, row_offset, thresholds);
}

int lq_debug_build(void) {
#ifdef LQ_DEBUG
  return 1;
#else
  return 0;
#endif
}

int lq_debug_flags(uint32_t* flags, int clear) {
  if (!flags) return LQ_ERR_ARG;
  if (!lq_debug_build()) return LQ_ERR_UNSUPPORTED;
  unsigned int v = 0;
  if (debug_flags(&v, clear != 0) != hipSuccess) return LQ_ERR_LAUNCH;
  *flags = v;
  return LQ_OK;
}

}  // extern "C"
