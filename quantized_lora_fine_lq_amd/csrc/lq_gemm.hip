// Layer kernels for gfx950: the fused dequant-GEMM with its LoRA segment
// (forward and the transposed backward for grad_X), the decode GEMV, and the
// skinny LoRA products t = X A^T, u = G B, dA = s u^T X, dB = s G^T t.
//
// QLoRA (Heng's Blog), introduction: h = dequant(W0_NF4) x + (alpha/r) B A x,
// W0 dequantized to BFloat16 when used; the optimizer updates only A and B.
#include <algorithm>

#include "lq_device.h"

namespace lq {
namespace {

// ===========================================================================
// Fused dequant-GEMM.
//
// out[m][c] = sum_k A[m][k] * Bt[c][k] over a main segment (Bt = W' forward,
// Bt = W'^T backward; produced from the packed NF4 codes, or copied from the
// bf16 weight that the codebook format's dequantization writes first) followed by a LoRA
// segment of 2r columns: A-side [hi(s*L) | lo(s*L)] with L = t (forward) or
// u (backward) split into two bfloat16 terms, Bt-side [Lb | Lb] with
// Lb = B (forward) or A^T (backward), both formed in the kernel from the
// float32 L and the bf16 adapter. hi + lo carries L to about 2^-17, so the
// LoRA term is computed at float32-like accuracy on the bf16 MFMA.
//
// Tile 256 x 128 x 64 per 512-thread workgroup (8 waves, two per SIMD, so
// one wave's MFMAs overlap the other's loads, dequantization and LDS
// traffic). Wave w owns rows [64 (w % 4), +64) and all 128 columns of the
// tile (2 x 4 MFMA 32x32x16 tiles) over one half of every 64-wide k-step
// (kh = w / 4); the two halves are summed at the end. Fragment traffic from
// LDS is 0.75 KB per MFMA. Per 64-wide k-step the A tile
// (rows of X or G) is staged in LDS with coalesced 16-byte loads, and the Bt
// tile is dequantized cooperatively -- each weight once per workgroup --
// into LDS. Both are double buffered; the global loads of step j are issued
// two steps ahead. Inside a k-step, lane (i, h) of a 32x32x16 MFMA takes
// k = 32h + 8s + e in sub-step s, a permutation of k that both operands share.
// ===========================================================================
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int PITCH = BK + 8;  // bf16 per LDS row: 144 bytes, conflict-free b128 access
constexpr int GEMM_THREADS = 512;

struct GemmParams {
  const uint16_t* A;   // [M, Kc] bf16, row stride Kc
  int64_t M, Ncols, Kc;
  const float* L;      // LoRA segment source, A-side: t (forward) or u (backward), float32 [M, r]
  const uint16_t* lb;  // Bt-side source: B [Ncols, r] (forward) or A [r, Ncols] (backward), bf16
  int r;
  float s;             // alpha / r
  int fwd;             // 1: Lb(n, j) = B[n][j]; 0: Lb(n, j) = A[j][n]
  int R2;              // 64 * ceil(2r / 64) columns of the LoRA segment
  int gm;              // M-tiles per group of the tile order
  void* out;           // [M, Ncols]
  QWeight w;
  Nf4Levels lv;
  const uint16_t* wbf; // dequantized weight [N, K] bf16 (codebook format), else null
};

__device__ __forceinline__ void zero(u32x4_t& v) { v = u32x4_t{0u, 0u, 0u, 0u}; }

// float -> (hi, lo) bfloat16 pair with hi + lo ~= v
__device__ __forceinline__ void split_bf16(float v, float& hi, float& lo) {
  hi = bf16lo_to_f32(pack_bf16x2(v, 0.0f));
  lo = v - hi;
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// ---- A tile (rows of X or G) through LDS ------------------------------------
// Thread t stages 16-byte chunk c = t % 8 of tile rows t/8 + 64q (q = 0..3):
// each global load instruction of a wave reads 8 whole 128-byte row segments.
// Rows past M repeat row M-1 (their outputs are never stored); a chunk past
// the end of the contraction reads column 0 instead (the Bt tile is zero
// there, so it adds nothing).
template <bool TAIL>
__device__ __forceinline__ void load_a_tile(const GemmParams& p, int it, const uint16_t* const (&ar)[4],
                                            u32x4_t (&r)[4]) {
  const int64_t col = (int64_t)it * BK + 8 * (threadIdx.x & 7);
  const int64_t off = (TAIL && col + 8 > p.Kc) ? 0 : col;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = ld16(ar[q] + off);
}
__device__ __forceinline__ void store_a_tile(uint16_t* sA, const u32x4_t (&r)[4]) {
  uint16_t* dst = sA + (threadIdx.x >> 3) * PITCH + 8 * (threadIdx.x & 7);
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4_t*>(dst + 64 * q * PITCH) = r[q];
}

// Bt tiles written by the backward NF4 producer keep 16-byte chunk q of
// row c at chunk q ^ bsw(c) (its LDS writes then hit 64 distinct banks);
// the other producers store chunks in place.
template <bool SWZ>
__device__ __forceinline__ int bsw(int c) { return SWZ ? (c >> 4) & 7 : 0; }

// 16 MFMAs of one half of a 64-wide step, both operands from LDS: wave tile
// 64 x 128 = [2 row tiles] x [4 col tiles] over sub-steps 2 kh and 2 kh + 1
// (the other wave of the pair takes the other half); all fragments of the
// half are read up front.
template <bool SWZ>
__device__ __forceinline__ void mfma_half(const uint16_t* sAt, const uint16_t* sBt, f32x16_t (&acc)[2][4],
                                          int wr, int kh, int li, int lh) {
  const uint16_t* abase = sAt + (64 * wr + li) * PITCH + 32 * lh + 16 * kh;
  const int q0 = 4 * lh + 2 * kh;   // the lane's chunk in sub-step 2 kh
  u32x4_t a[2][2], b[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) a[u][rt] = ld16(abase + 32 * rt * PITCH + 8 * u);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int c = 32 * ct + li;
      b[u][ct] = ld16(sBt + c * PITCH + 8 * ((q0 + u) ^ bsw<SWZ>(c)));
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[u][rt]), as_bf16x8(b[u][ct]),
                                                              acc[rt][ct], 0, 0, 0);
}

// ---- LoRA segment tiles -------------------------------------------------------
// Step jt covers segment columns c = 64 jt + [0, 64): column c < r holds
// hi(s L[m][c]) on the A side and Lb(n, c) on the Bt side, column r <= c < 2r
// holds lo(s L[m][c - r]) and Lb(n, c - r), the rest are zero. The A-side tile
// uses the main A tiles' thread mapping and row clamping; the Bt-side tile
// maps thread -> row t/4, columns 16 (t % 4) .. +16 (rows past Ncols repeat
// the last one: their outputs are never stored).
template <bool SWZ>
__device__ __forceinline__ void lora_tiles(const GemmParams& p, int jt, int64_t m0, int64_t n0,
                                           uint16_t* sA, uint16_t* sB) {
  const int cA = BK * jt + 8 * (threadIdx.x & 7);
  u32x4_t ra[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* lrow = p.L + min(m0 + (threadIdx.x >> 3) + 64 * q, p.M - 1) * p.r;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = cA + e;
      float x = 0.0f;
      if (c < 2 * p.r) {
        float hi, lo;
        split_bf16(p.s * lrow[c < p.r ? c : c - p.r], hi, lo);
        x = (c < p.r) ? hi : lo;
      }
      v[e] = x;
    }
    ra[q] = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
  const int64_t n = min(n0 + row, p.Ncols - 1);
  uint32_t h[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int c = BK * jt + 16 * qq + e;
    uint32_t x = 0;
    if (c < 2 * p.r) {
      const int j = c < p.r ? c : c - p.r;
      x = p.fwd ? p.lb[n * p.r + j] : p.lb[(int64_t)j * p.Ncols + n];
    }
    h[e] = x;
  }
  store_a_tile(sA, ra);
  *reinterpret_cast<u32x4_t*>(sB + row * PITCH + 8 * ((2 * qq) ^ bsw<SWZ>(row))) =
      u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  *reinterpret_cast<u32x4_t*>(sB + row * PITCH + 8 * ((2 * qq + 1) ^ bsw<SWZ>(row))) =
      u32x4_t{h[8] | (h[9] << 16), h[10] | (h[11] << 16), h[12] | (h[13] << 16), h[14] | (h[15] << 16)};
}

// ---- Bt producers -----------------------------------------------------------
// load() only issues global loads into members; store() decodes and writes
// the dequantized bf16 tile to LDS. Keeping arithmetic out of load() lets
// the loads stay in flight for a whole step.

// Block constant from the loaded parts: float32 (DQ = false) or
// fma(E4M3(q8), s2, mean) (DQ = true).
template <bool DQ>
__device__ __forceinline__ float const_of(float c0, uint32_t q8, float s2, float mean) {
  return DQ ? __builtin_fmaf(e4m3_decode(q8), s2, mean) : c0;
}

// Forward NF4: Bt[n][k] = W'[n0 + n][64 it + k]; thread -> row t/4,
// columns 16 (t % 4) .. +16 (8 code bytes, one block constant).
template <bool DQ>
struct ProdFwdNF4 {
  static constexpr bool kSwz = false;
  const uint8_t* crow;   // codes of the thread's row at its 16 columns
  int64_t blk0;          // block index of step 0
  uint32_t code[2];
  float c0, s2;
  uint32_t q8;
  float livef;           // 0 for a padding step past the end: tile of zeros
  __device__ void init(const GemmParams& p, int64_t n0) {
    const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
    const int64_t n = min(n0 + row, p.w.N - 1);   // rows past N: outputs never stored
    const int64_t e0 = n * p.w.K + 16 * qq;
    crow = p.w.codes + e0 / 2;
    blk0 = e0 >> 6;
  }
  __device__ void load(const GemmParams& p, int step, int nMain) {
    livef = step < nMain ? 1.0f : 0.0f;
    const int it = min(step, nMain - 1);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(crow + (int64_t)it * (BK / 2));
    code[0] = src[0];
    code[1] = src[1];
    const int64_t blk = blk0 + it;
    if (DQ) {
      q8 = p.w.qc.absmax_q[blk];
      s2 = p.w.qc.dq_scale[blk >> 8];
    } else {
      c0 = p.w.qc.absmax[blk];
    }
  }
  __device__ void store(const GemmParams& p, uint16_t* sB, const f32x2_t* sPair, float mean) {
    const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
    const float cp = const_of<DQ>(c0, q8, s2, mean) * livef;   // c * 0 = 0 (c is finite)
    f32x2_t q[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) q[b] = sPair[(code[b >> 2] >> (8 * (b & 3))) & 0xFFu];
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(sB + row * PITCH + 16 * qq);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      u32x4_t o;
#pragma unroll
      for (int b = 0; b < 4; ++b) o[b] = pack_bf16x2(q[4 * d + b].x * cp, q[4 * d + b].y * cp);
      dst[d] = o;
    }
  }
};

// Backward NF4: Bt[c][n] = W'[64 it + n][n0 + c] (the contraction runs over
// W's rows). Thread t of wave w -> rows 8 w + 2 (t % 4) + {0, 1} of the step
// and columns 8 cg .. +8 with cg = (t % 64) / 4 (4 code bytes per row, one
// block constant per row): a load instruction reads 4 whole 64-byte row
// segments and 8 block constants. Each LDS word pairs the two rows of a
// column; with the chunk swizzle bsw() the 64 words of a write instruction
// fall in 64 distinct banks. Rows past N contribute zero: their constant is
// forced to 0.
template <bool DQ>
struct ProdBwdNF4 {
  static constexpr bool kSwz = true;
  int64_t kcol;          // first of the thread's 8 columns
  uint32_t code[2];
  float c0[2], s2[2];
  uint32_t q8[2];
  float livef[2];
  __device__ void init(const GemmParams& p, int64_t n0) {
    const int cg = (threadIdx.x & 63) >> 2;
    kcol = min(n0 + 8 * cg, p.w.K - 8);   // columns past K: outputs never stored
  }
  __device__ void load(const GemmParams& p, int step, int nMain) {
    const int rp = 8 * (threadIdx.x >> 6) + 2 * (threadIdx.x & 3);   // first row of the pair in the step
    const int it = min(step, nMain - 1);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t nrow = (int64_t)it * BK + rp + rr;
      const bool ok = step < nMain && nrow < p.w.N;
      livef[rr] = ok ? 1.0f : 0.0f;
      const int64_t e0 = min(nrow, p.w.N - 1) * p.w.K + kcol;   // a valid row either way
      code[rr] = *reinterpret_cast<const uint32_t*>(p.w.codes + e0 / 2);
      const int64_t blk = e0 >> 6;
      if (DQ) {
        q8[rr] = p.w.qc.absmax_q[blk];
        s2[rr] = p.w.qc.dq_scale[blk >> 8];
      } else {
        c0[rr] = p.w.qc.absmax[blk];
      }
    }
  }
  __device__ void store(const GemmParams& p, uint16_t* sB, const f32x2_t* sPair, float mean) {
    const int w = threadIdx.x >> 6, pr = threadIdx.x & 3, cg = (threadIdx.x & 63) >> 2;
    float v[2][8];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const float cp = const_of<DQ>(c0[rr], q8[rr], s2[rr], mean) * livef[rr];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x2_t q = sPair[(code[rr] >> (8 * b)) & 0xFFu];   // columns 8cg + 2b, +1
        v[rr][2 * b] = q.x * cp;
        v[rr][2 * b + 1] = q.y * cp;
      }
    }
    // word of column c at rows 8w + 2pr, +1: chunk w of row c
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int c = 8 * cg + cc;
      *reinterpret_cast<uint32_t*>(sB + c * PITCH + 8 * (w ^ bsw<true>(c)) + 2 * pr) = pack_bf16x2(v[0][cc], v[1][cc]);
    }
  }
};

// Dequantized bfloat16 weight (the codebook format: its per-channel
// dequantization kernel writes W' first). Forward: Bt[n][k] = W'[n0 + n][64 it
// + k]; thread -> row t/4, columns 16 (t % 4) .. +16 (two 16-byte loads).
template <bool DQ>
struct ProdFwdBF16 {
  static constexpr bool kSwz = false;
  const uint16_t* src;
  u32x4_t v[2];
  bool live;
  __device__ void init(const GemmParams& p, int64_t n0) {
    const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
    const int64_t n = min(n0 + row, p.w.N - 1);   // rows past N: outputs never stored
    src = p.wbf + n * p.w.K + 16 * qq;
  }
  __device__ void load(const GemmParams& p, int step, int nMain) {
    live = step < nMain;
    const int it = min(step, nMain - 1);
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src + (int64_t)it * BK);
    v[0] = s[0];
    v[1] = s[1];
  }
  __device__ void store(const GemmParams& p, uint16_t* sB, const f32x2_t*, float) {
    const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(sB + row * PITCH + 16 * qq);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    dst[0] = live ? v[0] : z;
    dst[1] = live ? v[1] : z;
  }
};

// Backward over a dequantized bfloat16 weight: Bt[c][n] = W'[64 it + n][n0 + c].
// Thread -> rows 2 (t % 32) + {0, 1} of the step, columns 8 (t / 32) .. +8
// (one 16-byte load per row); each LDS word pairs the two rows of a column.
// Rows past N contribute zero.
template <bool DQ>
struct ProdBwdBF16 {
  static constexpr bool kSwz = false;
  int64_t kcol;
  u32x4_t v[2];
  bool ok[2];
  __device__ void init(const GemmParams& p, int64_t n0) {
    const int kq = threadIdx.x >> 5;
    kcol = min(n0 + 8 * kq, p.w.K - 8);   // columns past K: outputs never stored
  }
  __device__ void load(const GemmParams& p, int step, int nMain) {
    const int g = threadIdx.x & 31;
    const int it = min(step, nMain - 1);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t nrow = (int64_t)it * BK + 2 * g + rr;
      ok[rr] = step < nMain && nrow < p.w.N;
      v[rr] = *reinterpret_cast<const u32x4_t*>(p.wbf + min(nrow, p.w.N - 1) * p.w.K + kcol);
    }
  }
  __device__ void store(const GemmParams& p, uint16_t* sB, const f32x2_t*, float) {
    const int g = threadIdx.x & 31, kq = threadIdx.x >> 5;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const u32x4_t a = ok[0] ? v[0] : z, b = ok[1] ? v[1] : z;
    uint32_t* dst = reinterpret_cast<uint32_t*>(sB + (8 * kq) * PITCH + 2 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[(2 * j) * (PITCH / 2)] = (a[j] & 0xFFFFu) | (b[j] << 16);
      dst[(2 * j + 1) * (PITCH / 2)] = (a[j] >> 16) | (b[j] & 0xFFFF0000u);
    }
  }
};

template <class Prod, bool OUT_F32, bool TAIL>
__global__ __launch_bounds__(GEMM_THREADS) void k_dq_gemm(GemmParams p) {
  // one LDS object with the pair table first: at LDS address 0 a lookup
  // address is one shift of the code byte
  struct __attribute__((aligned(16))) Lds {
    f32x2_t pair[256];
    uint16_t a[2][BM * PITCH];
    uint16_t b[2][BN * PITCH];
  };
  __shared__ Lds lds;
  f32x2_t* sPair = lds.pair;
  uint16_t (*sA)[BM * PITCH] = lds.a;
  uint16_t (*sB)[BN * PITCH] = lds.b;
  if (threadIdx.x < 256) sPair[threadIdx.x] = f32x2_t{p.lv.q[threadIdx.x >> 4], p.lv.q[threadIdx.x & 15]};

  // XCD-aware tile order: the 8 XCDs take workgroups round robin, so each
  // XCD gets a contiguous range of logical tiles. Logical tiles run over
  // groups of p.gm M-tiles with the N-tiles outer inside a group, so the
  // workgroups resident on one XCD at a time share p.gm A row-tiles and a
  // run of consecutive weight tiles in that XCD's L2.
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tiles_n = (p.Ncols + BN - 1) / BN;
  const int64_t total = tiles_m * tiles_n;
  const int64_t b = blockIdx.x;
  const int64_t per = total / 8, rem = total % 8;
  const int64_t xcd = b % 8, local = b / 8;
  const int64_t logical = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int64_t group = (int64_t)p.gm * tiles_n;
  const int64_t first_m = (logical / group) * p.gm;
  const int64_t gm = min((int64_t)p.gm, tiles_m - first_m);
  const int64_t within = logical % group;
  const int64_t tm = first_m + within % gm, tn = within / gm;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wr = wave & 3, kh = wave >> 2;
  const int li = lane & 31, lh = lane >> 5;
  const float mean = p.w.qc.absmax ? 0.0f : *p.w.qc.dq_mean;
  const int nMain = (int)((p.Kc + BK - 1) / BK);
  const uint16_t* ar[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    ar[q] = p.A + min(m0 + (threadIdx.x >> 3) + 64 * q, p.M - 1) * p.Kc;

  f32x16_t acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0.0f;

  // Two register sets (producer state + A chunks) alternate: the data of
  // step j is loaded during step j-2, written to LDS buffer j%2 at the end of
  // step j-1, and multiplied in step j. One barrier per step. Every step
  // issues the same loads (indices are clamped; a step past the end yields a
  // zero Bt tile), so each step is one basic block.
  Prod pa, pb;
  pa.init(p, n0);
  pb.init(p, n0);
  u32x4_t ra[4], rb[4];
  __syncthreads();  // sPair and producer tables ready

  pa.load(p, 0, nMain);
  load_a_tile<TAIL>(p, 0, ar, ra);
  pb.load(p, 1, nMain);
  load_a_tile<TAIL>(p, min(1, nMain - 1), ar, rb);
  pa.store(p, sB[0], sPair, mean);
  store_a_tile(sA[0], ra);
  __syncthreads();
  for (int it = 0; it < nMain; it += 2) {
    pa.load(p, it + 2, nMain);
    load_a_tile<TAIL>(p, min(it + 2, nMain - 1), ar, ra);
    mfma_half<Prod::kSwz>(sA[0], sB[0], acc, wr, kh, li, lh);
    pb.store(p, sB[1], sPair, mean);
    store_a_tile(sA[1], rb);
    __syncthreads();
    pb.load(p, it + 3, nMain);
    load_a_tile<TAIL>(p, min(it + 3, nMain - 1), ar, rb);
    mfma_half<Prod::kSwz>(sA[1], sB[1], acc, wr, kh, li, lh);
    pa.store(p, sB[0], sPair, mean);
    store_a_tile(sA[0], ra);
    __syncthreads();
  }

  // LoRA segment (R2 = 64 ceil(2r / 64) columns) through the same LDS tiles
  const int nLora = p.R2 / BK;
  for (int jt = 0; jt < nLora; ++jt) {
    lora_tiles<Prod::kSwz>(p, jt, m0, n0, sA[0], sB[0]);
    __syncthreads();
    mfma_half<Prod::kSwz>(sA[0], sB[0], acc, wr, kh, li, lh);
    __syncthreads();
  }

  // The two waves of a pair hold partial sums over the two k halves: the
  // kh = 1 wave hands its accumulators over through LDS (the A buffers are
  // free now), one 32-row tile at a time, in the lane order it holds them
  // (four consecutive values per 16-byte access).
  float* sR = reinterpret_cast<float*>(&sA[0][0]);   // 4 waves x 64 floats x 64 lanes = 64 KB
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (kh == 1) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          *reinterpret_cast<f32x4_t*>(sR + (((wr * 4 + ct) * 4 + v4) * 64 + lane) * 4) =
              f32x4_t{acc[rt][ct][4 * v4], acc[rt][ct][4 * v4 + 1], acc[rt][ct][4 * v4 + 2], acc[rt][ct][4 * v4 + 3]};
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4_t o = *reinterpret_cast<const f32x4_t*>(sR + (((wr * 4 + ct) * 4 + v4) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rt][ct][4 * v4 + e] += o[e];
        }
    }
    __syncthreads();
  }

  // epilogue (kh = 0 waves): lane holds column li of each 32x32 tile, rows
  // 8(v/4) + 4lh + v%4. bfloat16 output with Ncols % 8 == 0: adjacent lanes
  // swap one value so each holds a column pair of one row, the tile goes
  // through LDS, and all threads store whole 16-byte row chunks.
  if (!OUT_F32 && p.Ncols % 8 == 0) {
    constexpr int CP = BN + 8;                 // 136 bf16 per staged row
    uint16_t* sC = &sA[0][0];                  // 256 x 136 x 2 B fits in sA
    if (kh == 0) {
      const bool odd = li & 1;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const float send = odd ? acc[rt][ct][v] : acc[rt][ct][v + 1];
            const float recv = dpp_f32<DPP_QUAD_XOR1>(send);
            const int row = 64 * wr + 32 * rt + 8 * (v >> 2) + 4 * lh + (v & 3) + (odd ? 1 : 0);
            const int col = 32 * ct + (li & ~1);
            const uint32_t pair = odd ? pack_bf16x2(recv, acc[rt][ct][v + 1]) : pack_bf16x2(acc[rt][ct][v], recv);
            *reinterpret_cast<uint32_t*>(sC + row * CP + col) = pair;
          }
    }
    __syncthreads();
    const int c = threadIdx.x & 15;
    const int64_t gcol = n0 + 8 * c;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = (threadIdx.x >> 4) + 32 * q;
      const int64_t grow = m0 + row;
      if (grow < p.M && gcol < p.Ncols)
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(p.out) + grow * p.Ncols + gcol) =
            *reinterpret_cast<const u32x4_t*>(sC + row * CP + 8 * c);
    }
    return;
  }
  if (kh != 0) return;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t col = n0 + 32 * ct + li;
      if (col >= p.Ncols) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 64 * wr + 32 * rt + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (row < p.M) {
          if (OUT_F32) reinterpret_cast<float*>(p.out)[row * p.Ncols + col] = acc[rt][ct][v];
          else reinterpret_cast<uint16_t*>(p.out)[row * p.Ncols + col] = (uint16_t)(pack_bf16x2(acc[rt][ct][v], 0.f) & 0xFFFFu);
        }
      }
    }
}

// ===========================================================================
// Decode GEMV (M <= 16), NF4. MFMA 16x16x32 with the tokens as the 16 A-rows
// (rows >= M repeat row M-1; their outputs are not stored) and 16 weight rows
// per MFMA tile. A workgroup owns RG row groups (16 RG weight rows); its 8
// waves split the K/128 stages evenly. In a stage, lane (li, lg) of row group
// g takes the 32 codes k = 32 lg + [0, 32) of row 16 g + li (one 16-byte
// load, inside one 64-block) and the same k of token li (from global
// memory, L2-resident; one X fragment serves all row groups). Codes are
// dequantized straight into MFMA B registers through a 256-entry LDS table
// of level pairs (one 8-byte lookup per code byte). The block constants of
// the workgroup's rows are decoded once into LDS at the start, so the main
// loop loads nothing but codes and X. The 8 partial sums are reduced in LDS
// at the end, where the LoRA term is added.
// ===========================================================================
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

constexpr int GV_WAVES = 8;        // K splits per workgroup
constexpr int GV_CTAB = 8448;      // floats of LDS for the constant table (33 KB: two workgroups per CU)
static_assert(GV_WAVES * 4 * 4 * 64 <= GV_CTAB, "the epilogue's partial sums of 4 row groups reuse the table");

// One pipeline stage: two 64-blocks (128 k) of RG row groups.
template <int RG>
struct GvStage {
  u32x4_t code[RG];      // 32 codes: k = 32 lg + [0, 32) of the stage
  u32x4_t x[4];          // X fragments, k = 32 lg + 8 u + [0, 8)
  int bl;                // the lane's block within the row
  float live;
};

template <int RG>
__device__ __forceinline__ void gv_load(const uint8_t* const (&crow)[RG], const uint16_t* xrow, int lg,
                                        int st2, int e1, int ns, int nb, GvStage<RG>& st) {
  // the lane's block: 2 ss + lg / 2 (past the row when K/64 is odd and this
  // is the last stage); its loads use a valid block either way and add 0
  const int ss = min(st2, ns - 1);
  const int bl = 2 * ss + (lg >> 1);
  st.live = (st2 < e1 && bl < nb) ? 1.0f : 0.0f;
  st.bl = min(bl, nb - 1);
#pragma unroll
  for (int g = 0; g < RG; ++g) st.code[g] = ld16(crow[g] + (int64_t)st.bl * 32 + 16 * (lg & 1));
  const uint16_t* xs = xrow + (int64_t)st.bl * 64 + 32 * (lg & 1);
#pragma unroll
  for (int u = 0; u < 4; ++u) st.x[u] = ld16(xs + 8 * u);
}

// 8 codes of one code word -> 8 bf16 through the LDS table of level pairs
// (high nibble = first level).
__device__ __forceinline__ u32x4_t dequant8_pair(uint32_t w, const f32x2_t* sPair, float cp) {
  u32x4_t o;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2_t q = sPair[(w >> (8 * b)) & 0xFFu];
    o[b] = pack_bf16x2(q.x * cp, q.y * cp);
  }
  return o;
}

// Sub-step outer, row group inner: consecutive MFMAs go to different
// accumulators, so none waits for the previous one.
template <int RG>
__device__ __forceinline__ void gv_compute(const GvStage<RG>& st, const f32x2_t* sPair, const float* sC,
                                           int pitch, int li, f32x4_t (&acc)[RG]) {
  float cp[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) cp[g] = sC[(16 * g + li) * pitch + st.bl] * st.live;   // c * 0 = 0
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const u32x4_t bv = dequant8_pair(st.code[g][u], sPair, cp[g]);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[u]), as_bf16x8(bv), acc[g], 0, 0, 0);
    }
}

template <int RG, bool DQ, bool OUT_F32>
__global__ __launch_bounds__(64 * GV_WAVES, 2) void k_gemv_nf4(GemvParams p) {
  // one LDS object with the pair table first: at LDS address 0 a lookup
  // address is one shift of the code byte
  struct __attribute__((aligned(16))) Lds {
    f32x2_t pair[256];
    float c[GV_CTAB];   // constants [16 RG rows][nb + 1]; then partial sums
  };
  __shared__ Lds lds;
  f32x2_t* sPair = lds.pair;
  float* sC = lds.c;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t N = p.w.N, K = p.w.K;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * RG;
  const int nb = (int)(K / 64);
  const int pitch = nb + 1;                // odd pitch: the 16 rows of a lookup hit distinct banks
  const int ns = (int)((K + 127) / 128);   // stages; the last one is half empty when nb is odd
  const int e0 = (int)((int64_t)wave * ns / GV_WAVES), e1 = (int)((int64_t)(wave + 1) * ns / GV_WAVES);

  const uint8_t* crow[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) crow[g] = p.w.codes + min(n0 + 16 * g + li, N - 1) * (K / 2);   // rows past N: not stored
  const uint16_t* xrow = p.X + min((int64_t)li, p.M - 1) * K;

  // first stage's loads go out before the constant table is built
  GvStage<RG> s0, s1;
  gv_load<RG>(crow, xrow, lg, e0, e1, ns, nb, s0);

  if (threadIdx.x < 256) sPair[threadIdx.x] = f32x2_t{p.lv.q[threadIdx.x >> 4], p.lv.q[threadIdx.x & 15]};
  const float mean = DQ ? *p.w.qc.dq_mean : 0.0f;
  if (DQ && nb % 16 == 0) {
    // 16 constants per thread and chunk: one 16-byte load of E4M3 codes and
    // one second-level scale (16 aligned blocks never straddle a 256-block),
    // all chunks of a thread in flight together
    const int cpr = nb / 16, nchunks = 16 * RG * cpr;
    constexpr int CH = (16 * RG * (GV_CTAB / (16 * RG) / 16) + 64 * GV_WAVES - 1) / (64 * GV_WAVES);
    u32x4_t q8[CH];
    float s2[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = min((int)threadIdx.x + u * 64 * GV_WAVES, nchunks - 1);
      const int rr = i / cpr, cb = i - rr * cpr;
      const int64_t blk = min(n0 + rr, N - 1) * nb + 16 * cb;
      q8[u] = ld16(p.w.qc.absmax_q + blk);
      s2[u] = p.w.qc.dq_scale[blk >> 8];
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int i = (int)threadIdx.x + u * 64 * GV_WAVES;
      if (i >= nchunks) continue;
      const int rr = i / cpr, cb = i - rr * cpr;
      float* dst = sC + rr * pitch + 16 * cb;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        dst[e] = __builtin_fmaf(e4m3_decode((q8[u][e >> 2] >> (8 * (e & 3))) & 0xFFu), s2[u], mean);
    }
  } else {
    const int ncon = 16 * RG * nb;
#pragma unroll 4
    for (int i = threadIdx.x; i < ncon; i += 64 * GV_WAVES) {
      const int rr = i / nb, bl = i - rr * nb;
      const int64_t blk = min(n0 + rr, N - 1) * nb + bl;
      const float c = DQ ? __builtin_fmaf(e4m3_decode(p.w.qc.absmax_q[blk]), p.w.qc.dq_scale[blk >> 8], mean)
                         : p.w.qc.absmax[blk];
      sC[rr * pitch + bl] = c;
    }
  }
  __syncthreads();

  f32x4_t acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The scheduling barriers keep each stage's loads where they are issued
  // (left alone, the compiler sinks them next to their first use and the
  // wave then waits for them).
  for (int st = e0; st < e1; st += 2) {
    gv_load<RG>(crow, xrow, lg, st + 1, e1, ns, nb, s1);
    __builtin_amdgcn_sched_barrier(0);
    gv_compute<RG>(s0, sPair, sC, pitch, li, acc);
    gv_load<RG>(crow, xrow, lg, st + 2, e1, ns, nb, s0);
    __builtin_amdgcn_sched_barrier(0);
    gv_compute<RG>(s1, sPair, sC, pitch, li, acc);
  }

  // reduce the 8 K-splits (the constant table is free now); lane (li, lg)
  // holds tokens 4 lg + v of row 16 g + li
  __syncthreads();
  float* sR = sC;   // [wave][group][v][lane]
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) sR[((wave * RG + g) * 4 + v) * 64 + lane] = acc[g][v];
  __syncthreads();
  for (int idx = threadIdx.x; idx < RG * 64; idx += 64 * GV_WAVES) {
    const int g = idx >> 6, ln = idx & 63;
    const int64_t n = n0 + 16 * g + (ln & 15);
    if (n >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * (ln >> 4) + v;
      if (m >= p.M) continue;
      float h = 0.0f;
#pragma unroll
      for (int w = 0; w < GV_WAVES; ++w) h += sR[((w * RG + g) * 4 + v) * 64 + ln];
      float lora = 0.0f;
      for (int j = 0; j < p.r; ++j) lora = __builtin_fmaf(p.t[m * p.r + j], bf16_to_f32(p.B[n * p.r + j]), lora);
      h += p.s * lora;
      if (OUT_F32) reinterpret_cast<float*>(p.out)[m * N + n] = h;
      else reinterpret_cast<uint16_t*>(p.out)[m * N + n] = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
    }
  }
}

// ===========================================================================
// Skinny products (HBM-bound: they stream X or G once).
// ===========================================================================
// Row form: out[m][j] = sum_c Q[m][c] R[j][c] with R [r, C] row-major (C a
// multiple of 8). One workgroup per 16 rows of Q; its W waves (16 for r <= 64,
// else 8) take contiguous runs of 64-column blocks. MFMA 16x16x32 with the
// contraction order permuted inside each 64-column block: in its two steps
// lane (li, lg) takes columns 16 lg + [0, 8) and 16 lg + [8, 16) of Q row li
// and of R row 16jt + li, straight into MFMA registers, so the four lanes of
// a row read whole 128-byte lines (R is small and stays in cache). The W
// partial sums meet in LDS and are added in wave order, so no second pass is
// needed. When pt2 is given, the result is also written split and
// transposed for the column form: pt2 [2r][Mp] bf16 = [hi(out)^T ;
// lo(out)^T], zero for rows M..Mp-1 (the grid then covers Mp rows).
template <int JT, int W>
__global__ __launch_bounds__(64 * W) void k_row_skinny(const uint16_t* __restrict__ Q, int64_t M, int64_t C,
                                                       const uint16_t* __restrict__ R, int r,
                                                       float* __restrict__ out, uint16_t* __restrict__ pt2,
                                                       int64_t Mp) {
  __shared__ f32x4_t sPart[W][JT][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const uint16_t* qrow = Q + min(row0 + li, M - 1) * C + 16 * lg;   // rows past M: not stored
  const uint16_t* rrow[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) rrow[jt] = R + (int64_t)min(16 * jt + li, r - 1) * C + 16 * lg;
  const int64_t blocks = (C + 63) / 64;
  const int64_t per = (blocks + W - 1) / W;
  const int64_t b_begin = min(blocks, wave * per), b_end = min(blocks, b_begin + per);
  f32x4_t acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int U = JT <= 2 ? 4 : (JT <= 4 ? 2 : 1);   // 64-column blocks with loads in flight together
  for (int64_t bk = b_begin; bk < b_end; bk += U) {
    u32x4_t a[U][2], b[U][2][JT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t cc = 64 * (bk + u) + 8 * h;   // + 16 lg in the row pointers
        const bool ok = bk + u < b_end && cc + 16 * lg + 8 <= C;
        const int64_t off = ok ? cc : -16 * lg;     // a lane past the end reads columns 0..7 and adds 0
        a[u][h] = ld16(qrow + off);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) b[u][h][jt] = ld16(rrow[jt] + off);
        if (!ok) zero(a[u][h]);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
          acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][h]), as_bf16x8(b[u][h][jt]), acc[jt], 0,
                                                            0, 0);
  }
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) sPart[wave][jt][lane] = acc[jt];
  __syncthreads();
  // thread -> (jt, lane) of the 16 x 16JT output: column j = 16jt + li,
  // rows 4lg + v
  for (int idx = threadIdx.x; idx < JT * 64; idx += 64 * W) {
    const int jt = idx >> 6, ln = idx & 63;
    const int j = 16 * jt + (ln & 15);
    if (j >= r) continue;
    f32x4_t sum = sPart[0][jt][ln];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const f32x4_t o = sPart[w][jt][ln];
#pragma unroll
      for (int v = 0; v < 4; ++v) sum[v] += o[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = row0 + 4 * (ln >> 4) + v;
      if (row < M) out[row * r + j] = sum[v];
      if (pt2 && row < Mp) {
        float hi = 0.0f, lo = 0.0f;
        if (row < M) split_bf16(sum[v], hi, lo);
        pt2[(int64_t)j * Mp + row] = (uint16_t)(pack_bf16x2(hi, 0.f) & 0xFFFFu);
        pt2[(int64_t)(j + r) * Mp + row] = (uint16_t)(pack_bf16x2(lo, 0.f) & 0xFFFFu);
      }
    }
  }
}

// Set-up of the backward in one launch: Bt = B^T ([N, r] -> [r, N]) for the
// row form u = G B, and pt2 = [hi(t)^T ; lo(t)^T] ([2r][Mp] bf16, zero for
// rows M..Mp-1) for the column form dB = s G^T t.
__global__ __launch_bounds__(256) void k_bwd_prep(const uint16_t* __restrict__ B, int64_t N, int r,
                                                  uint16_t* __restrict__ Bt, const float* __restrict__ t, int64_t M,
                                                  int64_t Mp, uint16_t* __restrict__ pt2) {
  const int64_t nb = N * r, nt = (int64_t)r * Mp;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nb + nt; i += (int64_t)gridDim.x * 256) {
    if (i < nb) {
      const int64_t n = i / r, j = i % r;
      Bt[j * N + n] = B[i];
    } else {
      const int64_t k = i - nb, j = k / Mp, m = k % Mp;
      float hi = 0.0f, lo = 0.0f;
      if (m < M) split_bf16(t[m * r + j], hi, lo);
      pt2[j * Mp + m] = (uint16_t)(pack_bf16x2(hi, 0.f) & 0xFFFFu);
      pt2[(j + r) * Mp + m] = (uint16_t)(pack_bf16x2(lo, 0.f) & 0xFFFFu);
    }
  }
}

// out[j][n] = in[n][j] for a small [N, r] bf16 matrix.
__global__ __launch_bounds__(256) void k_transpose_u16(const uint16_t* __restrict__ in, int64_t N, int r,
                                                       uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * r) return;
  const int64_t n = i / r, j = i % r;
  out[j * N + n] = in[i];
}

// Column form: out(j, c) = scale * sum_m P[m][j] Q[m][c] for j < r, P float32
// [M, r] small, Q bfloat16 [M, C] streamed once. P enters as pt2 = [hi(P)^T ;
// lo(P)^T] (bfloat16 [2r, Mp], Mp = M rounded up to 32, zero padded; hi + lo
// carries P to about 2^-17), so an MFMA A fragment is one 16-byte load. The
// Q tile [32 m x 128 c] goes through LDS and is gathered along m for the B
// fragments. Workgroup: 128 columns x one m-split, wave: 32 columns, MFMA
// 32x32x16 over the 2r product rows; hi and lo rows are added in registers
// when r % 32 == 0 or r == 16 (partner row in the same lane), otherwise both
// are kept. Each workgroup writes the partial sums of its m-split;
// k_reduce_splits2 adds them.
// One job of the column form: product pt2^T-by-Q over its m-splits, in
// `tiles` column tiles of 128.
struct ColJob {
  const uint16_t* pt2;
  const uint16_t* Q;
  int64_t C;
  int64_t m_per_split;
  int splits;
  unsigned tiles;
  float* part;
};

// Two jobs share one launch (same M and r): workgroups x < j0.tiles take
// job 0, the rest job 1; split rows y past a job's own split count exit.
template <int JT2>
__global__ __launch_bounds__(256) void k_col_skinny(ColJob j0, ColJob j1, int64_t Mp, int64_t M, int r,
                                                    int combine) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[32 * (128 + 8)];
  const bool second = blockIdx.x >= j0.tiles;
  const ColJob jb = second ? j1 : j0;
  if ((int)blockIdx.y >= jb.splits) return;   // the whole workgroup
  const uint16_t* __restrict__ pt2 = jb.pt2;
  const uint16_t* __restrict__ Q = jb.Q;
  const int64_t C = jb.C, m_per_split = jb.m_per_split;
  float* __restrict__ part = jb.part;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t c0 = (int64_t)(second ? blockIdx.x - j0.tiles : blockIdx.x) * 128;
  const int64_t m_begin = (int64_t)blockIdx.y * m_per_split;
  const int64_t m_end = min(M, m_begin + m_per_split);
  const int rows2 = 2 * r;
  f32x16_t acc[JT2];
#pragma unroll
  for (int jt = 0; jt < JT2; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.f;
  // A-fragment rows (rows past 2r read row 0: their products are not used)
  const uint16_t* arow[JT2];
#pragma unroll
  for (int jt = 0; jt < JT2; ++jt) {
    const int j = 32 * jt + li;
    arow[jt] = pt2 + (int64_t)(j < rows2 ? j : 0) * Mp + 8 * lh;
  }
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
    // pt2 is zero past M (padding) and rows of Q past m_end are zero in LDS
    u32x4_t af[2][JT2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int jt = 0; jt < JT2; ++jt) af[s][jt] = ld16(arow[jt] + mb + 16 * s);
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
      for (int jt = 0; jt < JT2; ++jt)
        acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[s][jt]), as_bf16x8(bv), acc[jt], 0, 0, 0);
    }
    __syncthreads();
  }
  const int64_t c = c0 + 32 * wave + li;
  const int srows = combine ? r : rows2;
  if (c < C) {
    float* dst = part + (int64_t)blockIdx.y * srows * C;
    if (combine) {
      // partner row j + r: tile jt + r/32 (r % 32 == 0) or v + 8 of the same tile (r == 16)
#pragma unroll
      for (int jt = 0; jt < JT2; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + 8 * (v >> 2) + 4 * lh + (v & 3);
          if (j >= r) continue;
          float partner = 0.0f;
          if (r == 16) partner = acc[jt][(v + 8) & 15];
#pragma unroll
          for (int pt = 0; pt < JT2; ++pt)
            if (r % 32 == 0 && pt == jt + r / 32) partner = acc[pt][v];
          dst[(int64_t)j * C + c] = acc[jt][v] + partner;
        }
    } else {
#pragma unroll
      for (int jt = 0; jt < JT2; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + 8 * (v >> 2) + 4 * lh + (v & 3);
          if (j < rows2) dst[(int64_t)j * C + c] = acc[jt][v];
        }
    }
  }
}

// Two split reductions in one launch (dB and dA of the backward): for each
// i < n1 + n2, out = scale * sum_s (part[s][i] + part[s][i + pair]) in split
// order, rows x cols per job, optionally written transposed ([cols, rows]).
struct SplitJob {
  const float* part;
  int splits;
  int64_t rows, cols, srows, pair;
  float scale;
  float* out;
  int transposed;
};

__device__ __forceinline__ void reduce_one(const SplitJob& jb, int64_t i) {
  const int64_t sn = jb.srows * jb.cols;
  const float* ps = jb.part + i;
  float acc = 0.0f;
  int s = 0;
  for (; s + 4 <= jb.splits; s += 4) {   // four loads in flight, added in order
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* q = ps + (int64_t)(s + u) * sn;
      v[u] = jb.pair ? q[0] + q[jb.pair] : q[0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += v[u];
  }
  for (; s < jb.splits; ++s) {
    const float* q = ps + (int64_t)s * sn;
    acc += jb.pair ? q[0] + q[jb.pair] : q[0];
  }
  acc *= jb.scale;
  if (jb.transposed) {
    const int64_t rr = i / jb.cols, cc = i % jb.cols;
    jb.out[cc * jb.rows + rr] = acc;
  } else {
    jb.out[i] = acc;
  }
}

__global__ __launch_bounds__(256) void k_reduce_splits2(SplitJob j1, SplitJob j2) {
  const int64_t n1 = j1.out ? j1.rows * j1.cols : 0;
  const int64_t n2 = j2.out ? j2.rows * j2.cols : 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n1 + n2; i += (int64_t)gridDim.x * 256) {
    if (i < n1) reduce_one(j1, i);
    else reduce_one(j2, i - n1);
  }
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

int64_t split_rows(int64_t M) { return (M + 31) / 32 * 32; }

hipError_t launch_row_skinny(const uint16_t* Q, int64_t M, int64_t C, const uint16_t* R, int r,
                             float* out, uint16_t* pt2, hipStream_t s) {
  const int64_t Mp = split_rows(M);
  const int64_t rows = pt2 ? Mp : M;
  const dim3 grid((unsigned)((rows + 15) / 16));
  switch ((r + 15) / 16) {
#define LQ_RS(JT, W) case JT: hipLaunchKernelGGL((k_row_skinny<JT, W>), grid, dim3(64 * W), 0, s, Q, M, C, R, r, out, pt2, Mp); break;
    LQ_RS(1, 16) LQ_RS(2, 16) LQ_RS(3, 16) LQ_RS(4, 16) LQ_RS(5, 8) LQ_RS(6, 8) LQ_RS(7, 8) LQ_RS(8, 8)
#undef LQ_RS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const uint16_t* B, int64_t N, int r, uint16_t* Bt, const float* t, int64_t M,
                           uint16_t* pt2, hipStream_t s) {
  const int64_t n = N * r + (int64_t)r * split_rows(M);
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(k_bwd_prep, dim3(blocks), dim3(256), 0, s, B, N, r, Bt, t, M, split_rows(M), pt2);
  return hipGetLastError();
}

hipError_t launch_transpose_u16(const uint16_t* in, int64_t N, int r, uint16_t* out, hipStream_t s) {
  const int64_t n = N * r;
  hipLaunchKernelGGL(k_transpose_u16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in, N, r, out);
  return hipGetLastError();
}

// workspace: partial sums [splits][2r][C] floats
size_t col_skinny_ws_floats(int64_t M, int64_t C, int r) {
  return (size_t)col_skinny_splits(M, C) * 2 * r * C;
}

// Partial sums of the column form into ws ([splits][srows][C]); returns the
// reduction job that finishes it (run by launch_reduce_splits2).
hipError_t launch_col_skinny(const ColSkinnyReq* a, const ColSkinnyReq* b, int64_t M, int r, SplitJobDesc* ja,
                             SplitJobDesc* jb, hipStream_t s) {
  const ColSkinnyReq* req[2] = {a, b};
  SplitJobDesc* desc[2] = {ja, jb};
  ColJob job[2] = {};
  int njobs = 0, ymax = 1;
  const int combine = (r % 32 == 0 || r == 16) ? 1 : 0;
  for (int i = 0; i < 2; ++i) {
    if (!req[i]) continue;
    const ColSkinnyReq& q = *req[i];
    const int splits = col_skinny_splits(M, q.C);
    const int64_t mchunks = (M + 31) / 32;
    const int64_t m_per_split = ((mchunks + splits - 1) / splits) * 32;
    const int real_splits = (int)((M + m_per_split - 1) / m_per_split);
    job[njobs] = ColJob{q.pt2, q.Q, q.C, m_per_split, real_splits, (unsigned)((q.C + 127) / 128), q.ws};
    ymax = std::max(ymax, real_splits);
    ++njobs;
    SplitJobDesc* d = desc[i];
    d->part = q.ws;
    d->splits = real_splits;
    d->rows = r;
    d->cols = q.C;
    d->srows = combine ? r : 2 * r;
    d->pair = combine ? 0 : (int64_t)r * q.C;
    d->scale = q.scale;
    d->out = q.out;
    d->transposed = q.out_transposed ? 1 : 0;
  }
  if (njobs == 0) return hipSuccess;
  const dim3 grid(job[0].tiles + (njobs > 1 ? job[1].tiles : 0u), (unsigned)ymax);
  switch ((2 * r + 31) / 32) {
#define LQ_CS(JT) case JT: hipLaunchKernelGGL(k_col_skinny<JT>, grid, dim3(256), 0, s, job[0], job[1], split_rows(M), M, r, combine); break;
    LQ_CS(1) LQ_CS(2) LQ_CS(3) LQ_CS(4) LQ_CS(5) LQ_CS(6) LQ_CS(7) LQ_CS(8)
#undef LQ_CS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce_splits2(const SplitJobDesc& a, const SplitJobDesc& b, hipStream_t s) {
  SplitJob j[2];
  const SplitJobDesc* d[2] = {&a, &b};
  int64_t n = 0;
  for (int i = 0; i < 2; ++i) {
    j[i] = SplitJob{d[i]->part, d[i]->splits, d[i]->rows, d[i]->cols, d[i]->srows, d[i]->pair, d[i]->scale,
                    d[i]->out, d[i]->transposed};
    if (d[i]->out) n += d[i]->rows * d[i]->cols;
  }
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(k_reduce_splits2, dim3(blocks), dim3(256), 0, s, j[0], j[1]);
  return hipGetLastError();
}

int lora_seg_cols(int r) { return BK * ((2 * r + BK - 1) / BK); }

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the forward / backward GEMM: (codebook format) the dequantized
// bf16 weight; none for NF4.
size_t gemm_ws_bytes(const QWeight& w, int64_t, int, bool) {
  return w.format == LQ_FMT_CODEBOOK ? align256((size_t)w.N * w.K * sizeof(uint16_t)) : 0;
}

// The LoRA segment's sources (read by the GEMM itself).
static void set_lora(GemmParams& p, const float* L, const uint16_t* lb, int r, float s, bool fwd) {
  p.L = L;
  p.lb = lb;
  p.r = r;
  p.s = s;
  p.fwd = fwd ? 1 : 0;
  p.R2 = lora_seg_cols(r);
}

static GemmParams make_params(const QWeight& w, const uint16_t* A, int64_t M, int64_t Ncols, int64_t Kc,
                              void* out) {
  GemmParams p;
  p.A = A; p.M = M; p.Ncols = Ncols; p.Kc = Kc; p.out = out;
  p.L = nullptr; p.lb = nullptr; p.r = 0; p.s = 0.0f; p.fwd = 1; p.R2 = 0;
  // 32 workgroups are resident per XCD: 2 A row-tiles x 16 weight tiles
  // minimise the bytes they pull into the XCD's L2.
  p.gm = (int)std::min<int64_t>(2, (M + BM - 1) / BM);
  p.w = w;
  p.lv = tables().lv;
  p.wbf = nullptr;
  return p;
}

hipError_t launch_gemm_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype, uint16_t* ws,
                           hipStream_t st) {
  GemmParams p = make_params(w, X, M, w.N, w.K, H);
  set_lora(p, t, B, r, s, true);
  hipError_t e = hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((w.N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  const bool dq = w.qc.absmax == nullptr;
  const bool f32 = h_dtype == LQ_F32;
#define LQ_LAUNCH_FWD(PROD)                                                                          \
  do {                                                                                               \
    if (dq && f32) hipLaunchKernelGGL((k_dq_gemm<PROD<true>, true, false>), grid, dim3(GEMM_THREADS), 0, st, p);   \
    else if (dq) hipLaunchKernelGGL((k_dq_gemm<PROD<true>, false, false>), grid, dim3(GEMM_THREADS), 0, st, p);    \
    else if (f32) hipLaunchKernelGGL((k_dq_gemm<PROD<false>, true, false>), grid, dim3(GEMM_THREADS), 0, st, p);   \
    else hipLaunchKernelGGL((k_dq_gemm<PROD<false>, false, false>), grid, dim3(GEMM_THREADS), 0, st, p);           \
  } while (0)
  if (w.format == LQ_FMT_NF4) {
    LQ_LAUNCH_FWD(ProdFwdNF4);
  } else {
    uint16_t* wbf = ws;
    e = launch_dequant(w, wbf, st);
    if (e != hipSuccess) return e;
    p.wbf = wbf;
    if (f32) hipLaunchKernelGGL((k_dq_gemm<ProdFwdBF16<false>, true, false>), grid, dim3(GEMM_THREADS), 0, st, p);
    else hipLaunchKernelGGL((k_dq_gemm<ProdFwdBF16<false>, false, false>), grid, dim3(GEMM_THREADS), 0, st, p);
  }
#undef LQ_LAUNCH_FWD
  return hipGetLastError();
}

hipError_t launch_gemm_bwd(const QWeight& w, const uint16_t* G, int64_t M, const float* u,
                           const uint16_t* A, int r, float s, uint16_t* gX, uint16_t* ws, hipStream_t st) {
  GemmParams p = make_params(w, G, M, w.K, w.N, gX);
  set_lora(p, u, A, r, s, false);
  hipError_t e = hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((w.K + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  const bool tail = w.N % BK != 0;   // contraction over N: last step partial
  if (w.format == LQ_FMT_CODEBOOK) {
    uint16_t* wbf = ws;
    e = launch_dequant(w, wbf, st);
    if (e != hipSuccess) return e;
    p.wbf = wbf;
    if (tail) hipLaunchKernelGGL((k_dq_gemm<ProdBwdBF16<false>, false, true>), grid, dim3(GEMM_THREADS), 0, st, p);
    else hipLaunchKernelGGL((k_dq_gemm<ProdBwdBF16<false>, false, false>), grid, dim3(GEMM_THREADS), 0, st, p);
  } else if (w.qc.absmax == nullptr) {
    if (tail) hipLaunchKernelGGL((k_dq_gemm<ProdBwdNF4<true>, false, true>), grid, dim3(GEMM_THREADS), 0, st, p);
    else hipLaunchKernelGGL((k_dq_gemm<ProdBwdNF4<true>, false, false>), grid, dim3(GEMM_THREADS), 0, st, p);
  } else {
    if (tail) hipLaunchKernelGGL((k_dq_gemm<ProdBwdNF4<false>, false, true>), grid, dim3(GEMM_THREADS), 0, st, p);
    else hipLaunchKernelGGL((k_dq_gemm<ProdBwdNF4<false>, false, false>), grid, dim3(GEMM_THREADS), 0, st, p);
  }
  return hipGetLastError();
}

// Row groups per workgroup: 4, 2 or 1, the largest whose constant table
// (16 RG rows of K/64 + 1 floats) fits in LDS and that still gives at least
// 1.5 workgroups per CU for M <= 4 (few loads per workgroup: latency wants
// more of them) or 1 per CU for larger M (more row groups per X fragment);
// 0 when not even one row group fits.
static int gemv_rg(int64_t N, int64_t K, int64_t M) {
  auto fits = [&](int rg) { return (int64_t)16 * rg * (K / 64 + 1) <= GV_CTAB; };
  const int64_t min_wgs = M <= 4 ? 384 : 256;
  int best = 0;
  for (int rg = 1; rg <= 4; rg *= 2) {
    if (!fits(rg)) break;
    if (best == 0 || (N + 16 * rg - 1) / (16 * rg) >= min_wgs) best = rg;
  }
  return best;
}

bool gemv_supported(const QWeight& w) {
  return w.format == LQ_FMT_NF4 && gemv_rg(w.N, w.K, 1) > 0;
}

template <int RG>
static void launch_gemv_rg(const GemvParams& p, bool dq, bool f32, hipStream_t st) {
  const dim3 grid((unsigned)((p.w.N + 16 * RG - 1) / (16 * RG))), block(64 * GV_WAVES);
  if (dq && f32) hipLaunchKernelGGL((k_gemv_nf4<RG, true, true>), grid, block, 0, st, p);
  else if (dq) hipLaunchKernelGGL((k_gemv_nf4<RG, true, false>), grid, block, 0, st, p);
  else if (f32) hipLaunchKernelGGL((k_gemv_nf4<RG, false, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((k_gemv_nf4<RG, false, false>), grid, block, 0, st, p);
}

hipError_t launch_gemv_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype,
                           hipStream_t st) {
  if (!gemv_supported(w)) return hipErrorInvalidValue;
  GemvParams p;
  p.X = X; p.M = M; p.t = t; p.B = B; p.r = r; p.s = s; p.out = H; p.w = w; p.lv = tables().lv;
  const bool dq = w.qc.absmax == nullptr, f32 = h_dtype == LQ_F32;
  const int rg = gemv_rg(w.N, w.K, M);
  if (rg == 4) launch_gemv_rg<4>(p, dq, f32, st);
  else if (rg == 2) launch_gemv_rg<2>(p, dq, f32, st);
  else launch_gemv_rg<1>(p, dq, f32, st);
  return hipGetLastError();
}

}  // namespace lq
