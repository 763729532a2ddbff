// Layer kernels for gfx950: the fused dequant-GEMM with its LoRA segment
// (forward and the transposed backward for grad_X), the decode GEMV, and the
// skinny LoRA products t = X A^T, u = G B, dA = s u^T X, dB = s G^T t.
//
// QLoRA (Heng's Blog), introduction: h = dequant(W0_NF4) x + (alpha/r) B A x,
// W0 dequantized to BFloat16 when used; the optimizer updates only A and B.
#include "lq_device.h"

namespace lq {
namespace {

// ===========================================================================
// Fused dequant-GEMM.
//
// out[m][c] = sum_k A[m][k] * Bt[c][k] over a main segment (Bt = W' forward,
// Bt = W'^T backward, both produced from packed codes) followed by a LoRA
// segment of 2r columns: A-side [hi(s*L) | lo(s*L)] with L = t (forward) or
// u (backward) split into two bfloat16 terms, Bt-side [Lb | Lb] with
// Lb = B (forward) or A^T (backward). hi + lo carries L to about 2^-17, so
// the LoRA term is computed at float32-like accuracy on the bf16 MFMA.
//
// Tile 256 x 128 x 64 per 256-thread workgroup; wave w owns rows
// [64w, 64w + 64) and all 128 columns (2 x 4 MFMA 32x32x16 tiles).
// The A operand goes straight from global memory into MFMA registers; the
// Bt tile is dequantized cooperatively (each weight once per workgroup)
// into a double-buffered LDS tile. Inside a 64-wide k-step, lane (i, h) of a
// 32x32x16 MFMA takes k = 32h + 8s + e for step s -- a permutation of k that
// both operands share, so each lane reads 64 contiguous bytes of A.
// ===========================================================================
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int PITCH = BK + 8;  // bf16 per LDS row: 144 bytes, conflict-free b128 access

struct GemmParams {
  const uint16_t* A;   // [M, Kc] bf16, row stride Kc
  int64_t M, Ncols, Kc;
  const float* la;     // [M, r] float32 (t or u)
  const uint16_t* lb;  // forward: B [N, r]; backward: A [r, K]
  int r;
  float s;
  void* out;           // [M, Ncols]
  QWeight w;
  Nf4Levels lv;
};

__device__ __forceinline__ void zero(u32x4_t& v) { v = u32x4_t{0u, 0u, 0u, 0u}; }

// float -> (hi, lo) bfloat16 pair with hi + lo ~= v
__device__ __forceinline__ void split_bf16(float v, float& hi, float& lo) {
  hi = bf16lo_to_f32(pack_bf16x2(v, 0.0f));
  lo = v - hi;
}

// A-side fragments of one k-step for one wave: [2 row tiles][4 sub-steps].
__device__ __forceinline__ void load_a_frags(const GemmParams& p, int it, int nMain, int64_t mrow0,
                                             int li, int lh, u32x4_t (&a)[2][4]) {
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t row = mrow0 + 32 * rt + li;
    const bool row_ok = row < p.M;
    if (it < nMain) {
      const uint16_t* src = p.A + row * p.Kc;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t col = (int64_t)it * BK + 32 * lh + 8 * s;
        if (row_ok && col + 8 <= p.Kc) {
          a[rt][s] = *reinterpret_cast<const u32x4_t*>(src + col);
        } else {
          zero(a[rt][s]);
          if (row_ok)
            for (int e = 0; e < 8; e += 2) {
              const uint32_t lo = (col + e < p.Kc) ? src[col + e] : 0u;
              const uint32_t hi = (col + e + 1 < p.Kc) ? src[col + e + 1] : 0u;
              a[rt][s][e / 2] = lo | (hi << 16);
            }
        }
      }
    } else {  // LoRA segment: columns [0, r) hi part, [r, 2r) lo part
      const float* src = p.la + row * p.r;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c0 = (it - nMain) * BK + 32 * lh + 8 * s;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + e;
          float x = 0.0f;
          if (row_ok && c < 2 * p.r) {
            float hi, lo;
            split_bf16(p.s * src[c < p.r ? c : c - p.r], hi, lo);
            x = (c < p.r) ? hi : lo;
          }
          v[e] = x;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) a[rt][s][e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      }
    }
  }
}

// ---- Bt producers -----------------------------------------------------------
// Forward NF4: Bt[n][k] = W'[n0 + n][64 it + k]; thread -> (row tid/2, 32 codes).
struct ProdFwdNF4 {
  __device__ void init(const GemmParams&, int64_t) {}
  u32x4_t codes;
  float cst;        // float32 constant, or decoded E4M3 value before the fma
  float s2;
  __device__ void load(const GemmParams& p, int it, int nMain, int64_t n0) {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t n = n0 + row;
    if (it < nMain) {
      if (n < p.w.N) {
        const int64_t e0 = n * p.w.K + (int64_t)it * BK + 32 * half;
        codes = *reinterpret_cast<const u32x4_t*>(p.w.codes + e0 / 2);
        const int64_t blk = e0 >> 6;
        if (p.w.qc.absmax) { cst = p.w.qc.absmax[blk]; s2 = 0.f; }
        else { cst = e4m3_decode(p.w.qc.absmax_q[blk]); s2 = p.w.qc.dq_scale[blk >> 8]; }
      } else {
        zero(codes); cst = 0.f; s2 = 0.f;
      }
    } else {  // LoRA segment: Bt[n][c] = B[n][c mod r] for c < 2r
      const int c0 = (it - nMain) * BK + 32 * half;
      uint32_t h[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int c = c0 + e;
        h[e] = (n < p.w.N && c < 2 * p.r) ? p.lb[n * p.r + (c < p.r ? c : c - p.r)] : 0u;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = h[8 * d + 2 * q] | (h[8 * d + 2 * q + 1] << 16);
        lora[d] = v;
      }
    }
  }
  u32x4_t lora[4];
  __device__ void store(const GemmParams& p, int it, int nMain, uint16_t* sB,
                        const f32x2_t* sPair, float mean) {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(sB + row * PITCH + 32 * half);
    if (it < nMain) {
      const float cp = p.w.qc.absmax ? cst : __builtin_fmaf(cst, s2, mean);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4_t o;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x2_t q = sPair[(codes[d] >> (8 * b)) & 0xFFu];
          o[b] = pack_bf16x2(q.x * cp, q.y * cp);
        }
        dst[d] = o;
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) dst[d] = lora[d];
    }
  }
};

// Backward NF4: Bt[c][n] = W'[64 it + n][n0 + c] (the contraction runs over
// W's rows). Thread -> 8 rows x 4 columns: g8 = tid % 8 picks rows
// 8*g8 .. 8*g8+7 of the 64-row step, kq = tid / 8 picks columns 4kq .. 4kq+3.
struct ProdBwdNF4 {
  __device__ void init(const GemmParams&, int64_t) {}
  uint32_t code16[8];   // 4 codes (2 bytes) per row
  float cst[8];
  float s2[8];
  u32x4_t lora[4];
  __device__ void load(const GemmParams& p, int it, int nMain, int64_t n0) {
    if (it < nMain) {
      const int g8 = threadIdx.x & 7, kq = threadIdx.x >> 3;
      const int64_t k = n0 + 4 * kq;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int64_t n = (int64_t)it * BK + 8 * g8 + rr;
        if (n < p.w.N && k < p.w.K) {
          const int64_t e0 = n * p.w.K + k;
          code16[rr] = *reinterpret_cast<const uint16_t*>(p.w.codes + e0 / 2);
          const int64_t blk = e0 >> 6;
          if (p.w.qc.absmax) { cst[rr] = p.w.qc.absmax[blk]; s2[rr] = 0.f; }
          else { cst[rr] = e4m3_decode(p.w.qc.absmax_q[blk]); s2[rr] = p.w.qc.dq_scale[blk >> 8]; }
        } else {
          code16[rr] = 0; cst[rr] = 0.f; s2[rr] = 0.f;
        }
      }
    } else {  // LoRA segment: Bt[c][j] = A[j mod r][n0 + c], thread -> (c = tid/2, 32 j)
      const int cl = threadIdx.x >> 1, half = threadIdx.x & 1;
      const int64_t kcol = n0 + cl;
      const int j0 = (it - nMain) * BK + 32 * half;
      uint32_t h[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int j = j0 + e;
        h[e] = (kcol < p.w.K && j < 2 * p.r) ? p.lb[(int64_t)(j < p.r ? j : j - p.r) * p.w.K + kcol] : 0u;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = h[8 * d + 2 * q] | (h[8 * d + 2 * q + 1] << 16);
        lora[d] = v;
      }
    }
  }
  __device__ void store(const GemmParams& p, int it, int nMain, uint16_t* sB,
                        const f32x2_t* sPair, float mean) {
    if (it < nMain) {
      const int g8 = threadIdx.x & 7, kq = threadIdx.x >> 3;
      float v[8][4];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float cp = p.w.qc.absmax ? cst[rr] : __builtin_fmaf(cst[rr], s2[rr], mean);
        const f32x2_t q0 = sPair[code16[rr] & 0xFFu];         // columns 4kq, 4kq+1
        const f32x2_t q1 = sPair[(code16[rr] >> 8) & 0xFFu];  // columns 4kq+2, 4kq+3
        v[rr][0] = q0.x * cp; v[rr][1] = q0.y * cp;
        v[rr][2] = q1.x * cp; v[rr][3] = q1.y * cp;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(v[2 * q][kk], v[2 * q + 1][kk]);
        *reinterpret_cast<u32x4_t*>(sB + (4 * kq + kk) * PITCH + 8 * g8) = o;
      }
    } else {
      const int cl = threadIdx.x >> 1, half = threadIdx.x & 1;
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(sB + cl * PITCH + 32 * half);
#pragma unroll
      for (int d = 0; d < 4; ++d) dst[d] = lora[d];
    }
  }
};

// Codebook forward: Bt[n][k] from the row's bit-planes and its 16-entry
// mapping (staged in LDS for the workgroup's 128 rows).
struct ProdFwdCodebook {
  uint32_t plane[4];
  float cst, s2;
  u32x4_t lora[4];
  __device__ static float* levels_lds() {
    __shared__ float sL[BN * 17];
    return sL;
  }
  __device__ void init(const GemmParams& p, int64_t n0) {
    float* sL = levels_lds();
    for (int idx = threadIdx.x; idx < BN * 16; idx += 256) {
      const int rr = idx / 16, q = idx % 16;
      const int64_t n = n0 + rr;
      sL[rr * 17 + q] = (n < p.w.N) ? p.w.levels[n * 16 + q] : 0.f;
    }
  }
  __device__ void load(const GemmParams& p, int it, int nMain, int64_t n0) {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t n = n0 + row;
    if (it < nMain) {
      if (n < p.w.N) {
        const int nb = min(max((int)p.w.row_bits[n], 1), 4);
        const uint8_t* src = p.w.codes + p.w.row_offset[n] + (int64_t)it * 8 * nb + 4 * half;
#pragma unroll
        for (int q = 0; q < 4; ++q) plane[q] = (q < nb) ? *reinterpret_cast<const uint32_t*>(src + 8 * q) : 0u;
        const int64_t blk = n * (p.w.K / 64) + it;
        if (p.w.qc.absmax) { cst = p.w.qc.absmax[blk]; s2 = 0.f; }
        else { cst = e4m3_decode(p.w.qc.absmax_q[blk]); s2 = p.w.qc.dq_scale[blk >> 8]; }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) plane[q] = 0u;
        cst = 0.f; s2 = 0.f;
      }
    } else {
      const int c0 = (it - nMain) * BK + 32 * half;
      uint32_t h[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int c = c0 + e;
        h[e] = (n < p.w.N && c < 2 * p.r) ? p.lb[n * p.r + (c < p.r ? c : c - p.r)] : 0u;
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = h[8 * d + 2 * q] | (h[8 * d + 2 * q + 1] << 16);
        lora[d] = v;
      }
    }
  }
  __device__ void store(const GemmParams& p, int it, int nMain, uint16_t* sB,
                        const f32x2_t* /*sPair*/, float mean) {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(sB + row * PITCH + 32 * half);
    if (it < nMain) {
      const float cp = p.w.qc.absmax ? cst : __builtin_fmaf(cst, s2, mean);
      const float* L = levels_lds() + row * 17;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4_t o;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float x[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int e = 8 * d + 2 * b + t;
            uint32_t code = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) code |= ((plane[q] >> e) & 1u) << q;
            x[t] = L[code] * cp;
          }
          o[b] = pack_bf16x2(x[0], x[1]);
        }
        dst[d] = o;
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) dst[d] = lora[d];
    }
  }
};

template <class Prod, bool OUT_F32>
__global__ __launch_bounds__(256) void k_dq_gemm(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * PITCH];
  __shared__ f32x2_t sPair[256];
  sPair[threadIdx.x] = f32x2_t{p.lv.q[threadIdx.x >> 4], p.lv.q[threadIdx.x & 15]};

  // XCD-aware tile order: the 8 XCDs take workgroups round robin, so give
  // each XCD a contiguous range of tiles, M-tiles fastest (they share the
  // same weight columns).
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tiles_n = (p.Ncols + BN - 1) / BN;
  const int64_t total = tiles_m * tiles_n;
  const int64_t b = blockIdx.x;
  const int64_t per = total / 8, rem = total % 8;
  const int64_t xcd = b % 8, local = b / 8;
  const int64_t logical = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int64_t tm = logical % tiles_m, tn = logical / tiles_m;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t mrow0 = m0 + 64 * wave;
  const float mean = p.w.qc.absmax ? 0.0f : *p.w.qc.dq_mean;

  const int nMain = (int)((p.Kc + BK - 1) / BK);
  const int nIter = nMain + (2 * p.r + BK - 1) / BK;

  f32x16_t acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0.0f;

  Prod prod;
  prod.init(p, n0);
  u32x4_t a_cur[2][4], a_nxt[2][4];
  __syncthreads();  // sPair and producer tables ready
  prod.load(p, 0, nMain, n0);
  load_a_frags(p, 0, nMain, mrow0, li, lh, a_cur);
  prod.store(p, 0, nMain, sB[0], sPair, mean);
  __syncthreads();

  for (int it = 0; it < nIter; ++it) {
    const bool has_next = it + 1 < nIter;
    if (has_next) {
      prod.load(p, it + 1, nMain, n0);
      load_a_frags(p, it + 1, nMain, mrow0, li, lh, a_nxt);
    }
    const uint16_t* cur = sB[it & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(cur + (32 * ct + li) * PITCH + 32 * lh + 8 * s);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a_cur[rt][s]), as_bf16x8(bv),
                                                                acc[rt][ct], 0, 0, 0);
      }
    }
    if (has_next) prod.store(p, it + 1, nMain, sB[(it + 1) & 1], sPair, mean);
    __syncthreads();
    if (has_next) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int s = 0; s < 4; ++s) a_cur[rt][s] = a_nxt[rt][s];
    }
  }

  // epilogue: lane holds column li of each 32x32 tile, rows 8(v/4) + 4lh + v%4
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t col = n0 + 32 * ct + li;
      if (col >= p.Ncols) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = mrow0 + 32 * rt + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (row < p.M) {
          if (OUT_F32) reinterpret_cast<float*>(p.out)[row * p.Ncols + col] = acc[rt][ct][v];
          else reinterpret_cast<uint16_t*>(p.out)[row * p.Ncols + col] = (uint16_t)(pack_bf16x2(acc[rt][ct][v], 0.f) & 0xFFFFu);
        }
      }
    }
}

// ===========================================================================
// Decode GEMV (M <= 16), NF4. MFMA 16x16x32 with tokens as the 16 A-rows
// (rows >= M are zero) and 16 weight rows per tile. Each workgroup owns 64
// weight rows; its 4 waves split K in 128-wide chunks; each lane streams 16
// bytes of codes per 16-row group per chunk and dequantizes straight into
// MFMA B-registers. Partial sums meet in LDS; the LoRA term s t B^T is added
// in float32 before the single rounding of H.
// ===========================================================================
constexpr int GV_RG = 4;

struct GemvParams {
  const uint16_t* X;   // [M, K]
  int64_t M;
  const float* t;      // [M, r]
  const uint16_t* B;   // [N, r]
  int r;
  float s;
  void* out;
  QWeight w;
  Nf4Levels lv;
};

template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemv_nf4(GemvParams p) {
  __shared__ f32x2_t sPair[256];
  __shared__ f32x4_t sRed[4][GV_RG][64];
  sPair[threadIdx.x] = f32x2_t{p.lv.q[threadIdx.x >> 4], p.lv.q[threadIdx.x & 15]};
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t N = p.w.N, K = p.w.K;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * GV_RG);
  const float mean = p.w.qc.absmax ? 0.0f : *p.w.qc.dq_mean;
  f32x4_t acc[GV_RG];
#pragma unroll
  for (int g = 0; g < GV_RG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t nChunks = (K + 127) / 128;
  for (int64_t ch = wave; ch < nChunks; ch += 4) {
    const int64_t kb = ch * 128 + 32 * lg;
    const bool k_ok = kb < K;   // K % 64 == 0: then kb + 32 <= K
    u32x4_t xa[4];
    if (k_ok && li < p.M) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p.X + li * K + kb);
#pragma unroll
      for (int s = 0; s < 4; ++s) xa[s] = src[s];
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) zero(xa[s]);
    }
    u32x4_t cw[GV_RG];
    float cp[GV_RG];
#pragma unroll
    for (int g = 0; g < GV_RG; ++g) {
      const int64_t n = n0 + 16 * g + li;
      if (k_ok && n < N) {
        const int64_t e0 = n * K + kb;
        cw[g] = *reinterpret_cast<const u32x4_t*>(p.w.codes + e0 / 2);
        const int64_t blk = e0 >> 6;
        cp[g] = p.w.qc.absmax ? p.w.qc.absmax[blk]
                              : __builtin_fmaf(e4m3_decode(p.w.qc.absmax_q[blk]), p.w.qc.dq_scale[blk >> 8], mean);
      } else {
        zero(cw[g]);
        cp[g] = 0.f;
      }
    }
#pragma unroll
    for (int g = 0; g < GV_RG; ++g) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4_t bv;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x2_t q = sPair[(cw[g][s] >> (8 * b)) & 0xFFu];
          bv[b] = pack_bf16x2(q.x * cp[g], q.y * cp[g]);
        }
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[s]), as_bf16x8(bv), acc[g], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GV_RG; ++g) sRed[wave][g][lane] = acc[g];
  __syncthreads();
  // thread -> (g = tid/64, lane): tokens 4*(lane/16) + v, weight row n0 + 16g + lane%16
  const int g = threadIdx.x >> 6;
  f32x4_t sum = sRed[0][g][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) sum += sRed[w][g][lane];
  const int64_t n = n0 + 16 * g + li;
  if (n >= N) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t m = 4 * lg + v;
    if (m >= p.M) continue;
    float lora = 0.0f;
    for (int j = 0; j < p.r; ++j) lora = __builtin_fmaf(p.t[m * p.r + j], bf16_to_f32(p.B[n * p.r + j]), lora);
    const float h = sum[v] + p.s * lora;
    if (OUT_F32) reinterpret_cast<float*>(p.out)[m * N + n] = h;
    else reinterpret_cast<uint16_t*>(p.out)[m * N + n] = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
  }
}

// ===========================================================================
// Skinny products (HBM-bound: they stream X or G once).
// ===========================================================================
// Row form: part[split][m][j] = sum_{c in split} Q[m][c] R(j, c), MFMA
// 16x16x32 with 16 rows of Q per wave, R staged in LDS as [j][64 c].
constexpr int RS_ROWS = 64;
__global__ __launch_bounds__(256) void k_row_skinny(const uint16_t* __restrict__ Q, int64_t M,
                                                    int64_t C, const uint16_t* __restrict__ Rm,
                                                    int r_transposed, int r, int64_t c_per_split,
                                                    float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sR[128 * PITCH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t m = (int64_t)blockIdx.x * RS_ROWS + 16 * wave + li;
  const int64_t c_begin = (int64_t)blockIdx.y * c_per_split;
  const int64_t c_end = min(C, c_begin + c_per_split);
  const int jtiles = (r + 15) / 16;
  f32x4_t acc[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t c0 = c_begin; c0 < c_end; c0 += 64) {
    // stage R(j, c0 .. c0+63) for j < 16*jtiles (zero outside)
    for (int idx = threadIdx.x; idx < 16 * jtiles * 64; idx += 256) {
      const int j = idx / 64, cc = idx % 64;
      const int64_t c = c0 + cc;
      uint16_t v = 0;
      if (j < r && c < c_end) v = r_transposed ? Rm[c * r + j] : Rm[(int64_t)j * C + c];
      sR[j * PITCH + cc] = v;
    }
    __syncthreads();
    u32x4_t a[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t c = c0 + 16 * lg + 8 * s;
      if (m < M && c + 8 <= c_end) a[s] = *reinterpret_cast<const u32x4_t*>(Q + m * C + c);
      else {
        zero(a[s]);
        if (m < M)
          for (int e = 0; e < 8; e += 2) {
            const uint32_t lo = (c + e < c_end) ? Q[m * C + c + e] : 0u;
            const uint32_t hi = (c + e + 1 < c_end) ? Q[m * C + c + e + 1] : 0u;
            a[s][e / 2] = lo | (hi << 16);
          }
      }
    }
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt < jtiles) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(sR + (16 * jt + li) * PITCH + 16 * lg + 8 * s);
          acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[s]), as_bf16x8(bv), acc[jt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  // D: lane holds column j = 16jt + li, rows 4lg + v
  float* dst = out + (int64_t)blockIdx.y * M * r;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    if (jt >= jtiles) continue;
    const int j = 16 * jt + li;
    if (j >= r) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = (int64_t)blockIdx.x * RS_ROWS + 16 * wave + 4 * lg + v;
      if (row < M) dst[row * r + j] = acc[jt][v];
    }
  }
}

// Column form: part[split][j][c] = sum_{m in split} P[m][j] Q[m][c], MFMA
// 32x32x16 with A = P^T (hi/lo bf16 split of float32 P) and B = Q, both
// gathered along m from LDS. Workgroup: 128 columns, wave: 32 columns.
__global__ __launch_bounds__(256) void k_col_skinny(const float* __restrict__ P,
                                                    const uint16_t* __restrict__ Q, int64_t M,
                                                    int64_t C, int r, int64_t m_per_split,
                                                    float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[32 * (128 + 8)];
  __shared__ float sP[32 * (128 + 1)];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * 128;
  const int64_t m_begin = (int64_t)blockIdx.y * m_per_split;
  const int64_t m_end = min(M, m_begin + m_per_split);
  const int jtiles = (r + 31) / 32;
  f32x16_t acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.f;
  for (int64_t mb = m_begin; mb < m_end; mb += 32) {
    for (int idx = threadIdx.x; idx < 32 * 16; idx += 256) {
      const int row = idx / 16, cc = (idx % 16) * 8;
      const int64_t m = mb + row, c = c0 + cc;
      u32x4_t v;
      zero(v);
      if (m < m_end) {
        if (c + 8 <= C) v = *reinterpret_cast<const u32x4_t*>(Q + m * C + c);
        else
          for (int e = 0; e < 8; e += 2) {
            const uint32_t lo = (c + e < C) ? Q[m * C + c + e] : 0u;
            const uint32_t hi = (c + e + 1 < C) ? Q[m * C + c + e + 1] : 0u;
            v[e / 2] = lo | (hi << 16);
          }
      }
      *reinterpret_cast<u32x4_t*>(sQ + row * (128 + 8) + cc) = v;
    }
    for (int idx = threadIdx.x; idx < 32 * r; idx += 256) {
      const int row = idx / r, j = idx % r;
      const int64_t m = mb + row;
      sP[row * (128 + 1) + j] = (m < m_end) ? P[m * r + j] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t bv;
      const int col = 32 * wave + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = sQ[(16 * s + 8 * lh + 2 * e) * (128 + 8) + col];
        const uint32_t hi = sQ[(16 * s + 8 * lh + 2 * e + 1) * (128 + 8) + col];
        bv[e] = lo | (hi << 16);
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt < jtiles) {
          const int j = 32 * jt + li;
          float vh[8], vl[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = (j < r) ? sP[(16 * s + 8 * lh + e) * (128 + 1) + j] : 0.f;
            split_bf16(x, vh[e], vl[e]);
          }
          u32x4_t ah, al;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ah[e] = pack_bf16x2(vh[2 * e], vh[2 * e + 1]);
            al[e] = pack_bf16x2(vl[2 * e], vl[2 * e + 1]);
          }
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bv), acc[jt], 0, 0, 0);
          acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), as_bf16x8(bv), acc[jt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  float* dst = out + (int64_t)blockIdx.y * r * C;
  const int64_t c = c0 + 32 * wave + li;
  if (c >= C) return;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    if (jt >= jtiles) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = 32 * jt + 8 * (v >> 2) + 4 * lh + (v & 3);
      if (j < r) dst[(int64_t)j * C + c] = acc[jt][v];
    }
  }
}

// out[i] = scale * sum_{s < splits} part[s][i] (fixed order); optional
// transposed write for [rows, cols] -> [cols, rows].
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ part, int splits,
                                                       int64_t rows, int64_t cols, float scale,
                                                       float* __restrict__ out, int transposed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = rows * cols;
  if (i >= n) return;
  float acc = part[i];
  for (int s = 1; s < splits; ++s) acc += part[(int64_t)s * n + i];
  acc *= scale;
  if (transposed) {
    const int64_t rr = i / cols, cc = i % cols;
    out[cc * rows + rr] = acc;
  } else {
    out[i] = acc;
  }
}

int row_skinny_splits(int64_t M, int64_t C) {
  const int64_t row_tiles = (M + RS_ROWS - 1) / RS_ROWS;
  const int64_t chunks = (C + 63) / 64;
  int64_t splits = (512 + row_tiles - 1) / row_tiles;
  if (splits > chunks) splits = chunks;
  if (splits < 1) splits = 1;
  return (int)splits;
}

int col_skinny_splits(int64_t M, int64_t C) {
  const int64_t col_tiles = (C + 127) / 128;
  const int64_t mchunks = (M + 31) / 32;
  int64_t splits = (512 + col_tiles - 1) / col_tiles;
  if (splits > mchunks) splits = mchunks;
  if (splits < 1) splits = 1;
  return (int)splits;
}

}  // namespace

size_t row_skinny_ws_floats(int64_t M, int64_t C, int r) {
  const int splits = row_skinny_splits(M, C);
  return splits > 1 ? (size_t)splits * M * r : 0;
}

hipError_t launch_row_skinny(const uint16_t* Q, int64_t M, int64_t C, const uint16_t* Rm,
                             bool r_transposed, int r, float* out, float* ws, hipStream_t s) {
  const int splits = row_skinny_splits(M, C);
  const int64_t chunks = (C + 63) / 64;
  const int64_t c_per_split = ((chunks + splits - 1) / splits) * 64;
  const int real_splits = (int)((C + c_per_split - 1) / c_per_split);
  float* dst = real_splits > 1 ? ws : out;
  const dim3 grid((unsigned)((M + RS_ROWS - 1) / RS_ROWS), (unsigned)real_splits);
  hipLaunchKernelGGL(k_row_skinny, grid, dim3(256), 0, s, Q, M, C, Rm, r_transposed ? 1 : 0, r,
                     c_per_split, dst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || real_splits == 1) return e;
  const int64_t n = M * r;
  hipLaunchKernelGGL(k_reduce_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws,
                     real_splits, M, (int64_t)r, 1.0f, out, 0);
  return hipGetLastError();
}

size_t col_skinny_ws_floats(int64_t M, int64_t C, int r) {
  return (size_t)col_skinny_splits(M, C) * r * C;
}

hipError_t launch_col_skinny(const float* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                             float scale, float* out, bool out_transposed, float* ws,
                             hipStream_t s) {
  const int splits = col_skinny_splits(M, C);
  const int64_t mchunks = (M + 31) / 32;
  const int64_t m_per_split = ((mchunks + splits - 1) / splits) * 32;
  const int real_splits = (int)((M + m_per_split - 1) / m_per_split);
  const dim3 grid((unsigned)((C + 127) / 128), (unsigned)real_splits);
  hipLaunchKernelGGL(k_col_skinny, grid, dim3(256), 0, s, P, Q, M, C, r, m_per_split, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)r * C;
  hipLaunchKernelGGL(k_reduce_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws,
                     real_splits, (int64_t)r, C, scale, out, out_transposed ? 1 : 0);
  return hipGetLastError();
}

static GemmParams make_params(const QWeight& w, const uint16_t* A, int64_t M, int64_t Ncols,
                              int64_t Kc, const float* la, const uint16_t* lb, int r, float s,
                              void* out) {
  GemmParams p;
  p.A = A; p.M = M; p.Ncols = Ncols; p.Kc = Kc;
  p.la = la; p.lb = lb; p.r = r; p.s = s; p.out = out;
  p.w = w;
  p.lv = tables().lv;
  return p;
}

hipError_t launch_gemm_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype,
                           hipStream_t st) {
  GemmParams p = make_params(w, X, M, w.N, w.K, t, B, r, s, H);
  const int64_t tiles = ((M + BM - 1) / BM) * ((w.N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  if (w.format == LQ_FMT_NF4) {
    if (h_dtype == LQ_F32) hipLaunchKernelGGL((k_dq_gemm<ProdFwdNF4, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_dq_gemm<ProdFwdNF4, false>), grid, dim3(256), 0, st, p);
  } else {
    if (h_dtype == LQ_F32) hipLaunchKernelGGL((k_dq_gemm<ProdFwdCodebook, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_dq_gemm<ProdFwdCodebook, false>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const QWeight& w, const uint16_t* G, int64_t M, const float* u,
                           const uint16_t* A, int r, float s, uint16_t* gX, hipStream_t st) {
  GemmParams p = make_params(w, G, M, w.K, w.N, u, A, r, s, gX);
  const int64_t tiles = ((M + BM - 1) / BM) * ((w.K + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  if (w.format == LQ_FMT_NF4) hipLaunchKernelGGL((k_dq_gemm<ProdBwdNF4, false>), grid, dim3(256), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemv_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype,
                           hipStream_t st) {
  GemvParams p;
  p.X = X; p.M = M; p.t = t; p.B = B; p.r = r; p.s = s; p.out = H; p.w = w; p.lv = tables().lv;
  const dim3 grid((unsigned)((w.N + 16 * GV_RG - 1) / (16 * GV_RG)));
  if (h_dtype == LQ_F32) hipLaunchKernelGGL(k_gemv_nf4<true>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_gemv_nf4<false>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace lq
