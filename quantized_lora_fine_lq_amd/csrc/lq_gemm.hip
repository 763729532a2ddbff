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
constexpr int kCusPerXcd = 32;   // MI355X: 8 XCDs of 32 CUs
constexpr int PITCH = BK + 8;  // bf16 per LDS row: 144 bytes, conflict-free b128 access
constexpr int GEMM_THREADS = 512;

// Split reductions of the backward (dB and dA): for each output i of a job,
// out = scale * sum_s (part[s][i] + part[s][i + pair]) in split order, rows x
// cols per job, optionally written transposed ([cols, rows]). Run by the
// grad_X GEMM's workgroups after their tiles, or by k_reduce_splits2 when
// there is no grad_X.
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

struct GemmParams {
  const uint16_t* A;   // [M, Kc] bf16, row stride Kc
  int64_t M, Ncols, Kc;
  const float* L;      // LoRA segment source, A-side: t (forward) or u (backward), float32 [M, r]
  const uint16_t* lb;  // Bt-side source: B [Ncols, r] (forward) or A [r, Ncols] (backward), bf16
  int r;
  float s;             // alpha / r
  int fwd;             // 1: Lb(n, j) = B[n][j]; 0: Lb(n, j) = A[j][n]
  int lvec;            // 1: r % 8 == 0 and L 16-byte aligned (the segment tiles use 16-byte loads)
  int R2;              // 64 * ceil(2r / 64) columns of the LoRA segment
  int gm;              // M-tiles per group of the tile order
  void* out;           // [M, Ncols]
  QWeight w;
  Nf4Levels lv;
  const uint16_t* wbf; // dequantized weight [N, K] bf16 (codebook format), else null
  SplitJob red[2];     // split reductions to run after the tiles (backward), n = rows * cols each
  int64_t red_n[2];    // 0: none
  int cpx;             // CUs per XCD when the last tiles of each XCD are split in two k-halves, else 0
  float* part;         // the split tiles' float32 partial sums, [2 per split tile][BM][BN]
};

// ---- tile schedule ------------------------------------------------------------
// The 8 XCDs take workgroups round robin (workgroup b runs on XCD b % 8), and
// each XCD owns a contiguous range of logical tiles. One workgroup fills a CU,
// so an XCD of cpx CUs runs its tiles in rounds of cpx; when its last round
// would be at most half full, its last tiles are each split into two
// k-halves (twice as many workgroups, each half as long) whose float32
// partial sums a second kernel adds. Workgroup b takes item b / 8 of XCD b % 8.
__host__ __device__ inline int64_t xcd_tiles(int64_t total, int x) { return total / 8 + (x < total % 8 ? 1 : 0); }
__host__ __device__ inline int64_t xcd_first(int64_t total, int x) {
  return x * (total / 8) + (x < total % 8 ? x : total % 8);
}
__host__ __device__ inline int64_t xcd_splits(int64_t n_x, int cpx) {
  if (cpx <= 0 || n_x < cpx) return 0;
  const int64_t r = n_x % cpx;
  return 2 * r <= cpx ? r : 0;
}
// Logical tile -> (M-tile, N-tile): groups of gm M-tiles with the N-tiles
// outer inside a group, so the workgroups resident on one XCD at a time share
// gm A row-tiles and a run of consecutive weight tiles in that XCD's L2.
__host__ __device__ inline void tile_coords(int64_t t, int64_t tiles_m, int64_t tiles_n, int gm0, int64_t& tm,
                                            int64_t& tn) {
  const int64_t group = (int64_t)gm0 * tiles_n;
  const int64_t first_m = (t / group) * gm0;
  const int64_t gm = tiles_m - first_m < gm0 ? tiles_m - first_m : gm0;
  const int64_t within = t % group;
  tm = first_m + within % gm;
  tn = within / gm;
}

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
//
// Segment column c reads element seg_src(c, r) of its row: c, c - r, or 0
// for a zero column (a valid element either way, zeroed afterwards), so no
// load sits behind a branch. With r % 8 == 0 an aligned run of 8 segment
// columns lies inside one part (hi, lo or zero) and is 8 consecutive elements
// of the row, read as 16-byte loads when the rows are 16-byte aligned
// (lvec: L, and B's rows in the forward). On this GPU 4-byte loads of whole
// 256- and 512-byte rows (r = 64, 128) cost 10 us and more per step.
__device__ __forceinline__ int seg_src(int c, int r) { return c < r ? c : (c < 2 * r ? c - r : 0); }

template <bool SWZ>
__device__ __forceinline__ void lora_tiles(const GemmParams& p, int jt, int64_t m0, int64_t n0,
                                           uint16_t* sA, uint16_t* sB) {
  const int cA = BK * jt + 8 * (threadIdx.x & 7);
  float lv[4][8];
  if (p.lvec) {
    const int off = seg_src(cA, p.r);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* lrow = p.L + min(m0 + (threadIdx.x >> 3) + 64 * q, p.M - 1) * p.r + off;
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(lrow);
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(lrow + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lv[q][e] = v0[e];
        lv[q][4 + e] = v1[e];
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* lrow = p.L + min(m0 + (threadIdx.x >> 3) + 64 * q, p.M - 1) * p.r;
#pragma unroll
      for (int e = 0; e < 8; ++e) lv[q][e] = lrow[seg_src(cA + e, p.r)];
    }
  }
  const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
  const int64_t n = min(n0 + row, p.Ncols - 1);
  const int cB = BK * jt + 16 * qq;
  u32x4_t hb[2];
  if (p.fwd && p.lvec) {
    // B[n][.]: 8 bf16 of one part per 16-byte load, already in the tile's word order
    const uint16_t* brow = p.lb + n * p.r;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) hb[hh] = ld16(brow + seg_src(cB + 8 * hh, p.r));
  } else {
    // Lb(n, j): B[n][j] (row n of B, stride 1) or A[j][n] (column n of A, stride Ncols)
    const uint16_t* lbn = p.lb + (p.fwd ? n * p.r : n);
    const int64_t lbs = p.fwd ? 1 : p.Ncols;
    uint32_t h[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) h[e] = lbn[seg_src(cB + e, p.r) * lbs];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      hb[hh] = u32x4_t{h[8 * hh] | (h[8 * hh + 1] << 16), h[8 * hh + 2] | (h[8 * hh + 3] << 16),
                       h[8 * hh + 4] | (h[8 * hh + 5] << 16), h[8 * hh + 6] | (h[8 * hh + 7] << 16)};
  }
  u32x4_t ra[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = cA + e;
      float hi, lo;
      split_bf16(p.s * lv[q][e], hi, lo);
      v[e] = c < p.r ? hi : (c < 2 * p.r ? lo : 0.0f);
    }
    ra[q] = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  // zero columns (c >= 2r) of the Bt side, 16-bit element by element
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = cB + 8 * hh + 2 * w;
      const uint32_t keep = (c < 2 * p.r ? 0x0000FFFFu : 0u) | (c + 1 < 2 * p.r ? 0xFFFF0000u : 0u);
      hb[hh][w] &= keep;
    }
  store_a_tile(sA, ra);
  *reinterpret_cast<u32x4_t*>(sB + row * PITCH + 8 * ((2 * qq) ^ bsw<SWZ>(row))) = hb[0];
  *reinterpret_cast<u32x4_t*>(sB + row * PITCH + 8 * ((2 * qq + 1) ^ bsw<SWZ>(row))) = hb[1];
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
  __device__ void init(const GemmParams& p, int64_t n0, int ks) {
    const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
    const int64_t n = min(n0 + row, p.w.N - 1);   // rows past N: outputs never stored
    const int64_t e0 = n * p.w.K + 16 * qq + (int64_t)ks * BK;
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
  int ks;                // first step of this workgroup's range of the contraction
  uint32_t code[2];
  float c0[2], s2[2];
  uint32_t q8[2];
  float livef[2];
  __device__ void init(const GemmParams& p, int64_t n0, int ks0) {
    const int cg = (threadIdx.x & 63) >> 2;
    kcol = min(n0 + 8 * cg, p.w.K - 8);   // columns past K: outputs never stored
    ks = ks0;
  }
  __device__ void load(const GemmParams& p, int step, int nMain) {
    const int rp = 8 * (threadIdx.x >> 6) + 2 * (threadIdx.x & 3);   // first row of the pair in the step
    const int it = ks + min(step, nMain - 1);
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
  __device__ void init(const GemmParams& p, int64_t n0, int ks) {
    const int row = threadIdx.x >> 2, qq = threadIdx.x & 3;
    const int64_t n = min(n0 + row, p.w.N - 1);   // rows past N: outputs never stored
    src = p.wbf + n * p.w.K + 16 * qq + (int64_t)ks * BK;
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
  int ks;
  u32x4_t v[2];
  bool ok[2];
  __device__ void init(const GemmParams& p, int64_t n0, int ks0) {
    const int kq = threadIdx.x >> 5;
    kcol = min(n0 + 8 * kq, p.w.K - 8);   // columns past K: outputs never stored
    ks = ks0;
  }
  __device__ void load(const GemmParams& p, int step, int nMain) {
    const int g = threadIdx.x & 31;
    const int it = ks + min(step, nMain - 1);
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

// The split reductions handed to this launch, grid-stride over all its
// threads (each thread calls this exactly once, after its tile work).
__device__ __forceinline__ void gemm_reduce_tail(const GemmParams& p) {
  const int64_t n = p.red_n[0] + p.red_n[1];
  for (int64_t i = (int64_t)blockIdx.x * GEMM_THREADS + threadIdx.x; i < n; i += (int64_t)gridDim.x * GEMM_THREADS) {
    if (i < p.red_n[0]) reduce_one(p.red[0], i);
    else reduce_one(p.red[1], i - p.red_n[0]);
  }
}

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

  // this workgroup's item of its XCD's schedule: a whole tile, or one k-half
  // (half 0 or 1) of split tile number sidx
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tiles_n = (p.Ncols + BN - 1) / BN;
  const int64_t total = tiles_m * tiles_n;
  const int xcd = (int)(blockIdx.x % 8);
  const int64_t local = blockIdx.x / 8;
  const int64_t n_x = xcd_tiles(total, xcd), s_x = xcd_splits(n_x, p.cpx);
  if (local >= n_x + s_x) {   // past this XCD's items (the grid is 8 x the longest list)
    gemm_reduce_tail(p);
    return;
  }
  const int64_t whole = n_x - s_x;
  int64_t logical = xcd_first(total, xcd) + local, sidx = 0;
  int half = -1;
  if (local >= whole) {
    const int64_t j = local - whole;
    logical = xcd_first(total, xcd) + whole + j / 2;
    half = (int)(j & 1);
    for (int x = 0; x < xcd; ++x) sidx += xcd_splits(xcd_tiles(total, x), p.cpx);
    sidx += j / 2;
  }
  int64_t tm, tn;
  tile_coords(logical, tiles_m, tiles_n, p.gm, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int nK = (int)((p.Kc + BK - 1) / BK);
  const int ks = half == 1 ? nK / 2 : 0;                      // first step of this item
  const int nMain = half < 0 ? nK : (half == 0 ? nK / 2 : nK - nK / 2);

  if (threadIdx.x < 256) sPair[threadIdx.x] = f32x2_t{p.lv.q[threadIdx.x >> 4], p.lv.q[threadIdx.x & 15]};
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wr = wave & 3, kh = wave >> 2;
  const int li = lane & 31, lh = lane >> 5;
  const float mean = p.w.qc.absmax ? 0.0f : *p.w.qc.dq_mean;
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
  pa.init(p, n0, ks);
  pb.init(p, n0, ks);
  u32x4_t ra[4], rb[4];
  __syncthreads();  // sPair and producer tables ready

  pa.load(p, 0, nMain);
  load_a_tile<TAIL>(p, ks, ar, ra);
  pb.load(p, 1, nMain);
  load_a_tile<TAIL>(p, ks + min(1, nMain - 1), ar, rb);
  pa.store(p, sB[0], sPair, mean);
  store_a_tile(sA[0], ra);
  __syncthreads();
  for (int it = 0; it < nMain; it += 2) {
    pa.load(p, it + 2, nMain);
    load_a_tile<TAIL>(p, ks + min(it + 2, nMain - 1), ar, ra);
    mfma_half<Prod::kSwz>(sA[0], sB[0], acc, wr, kh, li, lh);
    pb.store(p, sB[1], sPair, mean);
    store_a_tile(sA[1], rb);
    __syncthreads();
    pb.load(p, it + 3, nMain);
    load_a_tile<TAIL>(p, ks + min(it + 3, nMain - 1), ar, rb);
    mfma_half<Prod::kSwz>(sA[1], sB[1], acc, wr, kh, li, lh);
    pa.store(p, sB[0], sPair, mean);
    store_a_tile(sA[0], ra);
    __syncthreads();
  }

  // LoRA segment (R2 = 64 ceil(2r / 64) columns) through the same LDS tiles;
  // of a split tile, only the first half adds it
  const int nLora = half == 1 ? 0 : p.R2 / BK;
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

  // a split tile's half: float32 partial sums, [BM][BN] row-major
  if (half >= 0) {
    if (kh == 0) {
      float* dst = p.part + (2 * sidx + half) * (int64_t)(BM * BN);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            dst[(64 * wr + 32 * rt + 8 * (v >> 2) + 4 * lh + (v & 3)) * BN + 32 * ct + li] = acc[rt][ct][v];
    }
    gemm_reduce_tail(p);
    return;
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
    gemm_reduce_tail(p);
    return;
  }
  if (kh != 0) {
    gemm_reduce_tail(p);
    return;
  }
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
  gemm_reduce_tail(p);
}

// The split tiles' two k-halves added (half 0 + half 1, in that order) and
// stored; thread -> 4 consecutive columns of one row of one split tile.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_split_fixup(GemmParams p, int64_t n_split) {
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tiles_n = (p.Ncols + BN - 1) / BN;
  const int64_t total = tiles_m * tiles_n;
  constexpr int PER_TILE = BM * BN / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_split * PER_TILE; i += (int64_t)gridDim.x * 256) {
    const int64_t sidx = i / PER_TILE;
    const int e = (int)(i % PER_TILE);
    // the split tile's logical index: its XCD's range, last s_x tiles
    int64_t base = 0, logical = 0;
    for (int x = 0; x < 8; ++x) {
      const int64_t n_x = xcd_tiles(total, x), s_x = xcd_splits(n_x, p.cpx);
      if (sidx < base + s_x) {
        logical = xcd_first(total, x) + n_x - s_x + (sidx - base);
        break;
      }
      base += s_x;
    }
    int64_t tm, tn;
    tile_coords(logical, tiles_m, tiles_n, p.gm, tm, tn);
    const int row = e / (BN / 4), col = 4 * (e % (BN / 4));
    const int64_t grow = tm * BM + row, gcol = tn * BN + col;
    if (grow >= p.M) continue;
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p.part + (2 * sidx) * (int64_t)(BM * BN) + row * BN + col);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p.part + (2 * sidx + 1) * (int64_t)(BM * BN) + row * BN + col);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (gcol + c >= p.Ncols) break;
      const float v = a[c] + b[c];
      if (OUT_F32) reinterpret_cast<float*>(p.out)[grow * p.Ncols + gcol + c] = v;
      else reinterpret_cast<uint16_t*>(p.out)[grow * p.Ncols + gcol + c] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
    }
  }
}

// ===========================================================================
// Decode GEMV (M <= 16), NF4. MFMA 16x16x32 with the tokens as the 16 A-rows
// (rows >= M repeat row M-1; their outputs are not stored) and 16 weight rows
// per MFMA tile. A workgroup owns RG row groups (16 RG weight rows); its 8
// waves share the K/128 stages. In a stage, lane (li, lg) of row group
// g takes the 32 codes k = 32 lg + [0, 32) of row 16 g + li (one 16-byte
// load, inside one 64-block) and the same k of token li (from global
// memory, L2-resident; one X fragment serves all row groups). Wave w takes
// stages w, w + 8, w + 16, ... Codes are
// dequantized straight into MFMA B registers through a 256-entry LDS table
// of level pairs (one 8-byte lookup per code byte). The block constants of
// the workgroup's rows are decoded once into LDS at the start, so the main
// loop loads nothing but codes and X. The LoRA term enters the accumulators
// as one more MFMA step per wave before the main loop, so the 8 partial sums
// reduced in LDS at the end are the whole result.
// ===========================================================================
struct GemvParams {
  const uint16_t* X;   // [M, K]
  int64_t M;
  const float* t;      // [M, r] as tparts partial sums [tparts][M][r], or null when the kernel forms
                       // t = X A^T itself
  int tparts;
  const uint16_t* B;   // [N, r]
  int r;
  float s;
  void* out;
  QWeight w;
  Nf4Levels lv;
  const uint16_t* A;   // [r, K] (t formed in the kernel)
  float* t_out;        // [M, r]: t, written by workgroup 0 (formed in the kernel, or summed from
                       // tparts > 1 partial sums), or null
};

// t = X A^T inside the NF4 decode kernel, for r <= GV_TR: every workgroup
// forms it over the same stages as its main loop (wave w: stages w, w + 8,
// ..., the X fragments of the main loop's layout and the matching 8-element
// pieces of A's rows as the MFMA's second operand), the 8 waves' partial sums
// are added in wave order in LDS, and the LoRA term is formed from that t.
// One launch instead of two for the whole forward at decode sizes.
constexpr int GV_TR = 32;

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

// The LoRA term of a GEMV tile on the matrix cores: s t B^T is the product of
// the segment [hi(s t) | lo(s t)] (2r columns, bfloat16 hi + lo ~= s t) with
// [B | B], taken in 32-column chunks, chunk w by wave w (r <= 128: at most 8
// chunks). Lane (li, lg) supplies token li (rows past M repeat row M - 1)
// and weight row `row` at columns 32 w + 8 lg + [0, 8); columns past 2r
// are zero. Waves whose whole chunk lies past 2r skip the loads (a
// wave-uniform test, gv_lora_live) and add nothing. Every load reads a valid
// element (a zero column reads column 0 and is masked after), so none sits
// behind a branch: the compiler would otherwise wait for each guarded load
// inside its branch, one latency per element. gv_lora_mfma adds the chunk to
// the wave's accumulator.
struct GvLora {
  u32x4_t a, b;
};
__device__ __forceinline__ bool gv_lora_live(int wave, int r) { return 32 * wave < 2 * r; }
__device__ __forceinline__ GvLora gv_lora_load(const float* t, const uint16_t* B, int64_t M, int r, float s,
                                               int wave, int li, int lg, int64_t row) {
  const float* trow = t + min((int64_t)li, M - 1) * r;
  const uint16_t* brow = B + row * r;
  float tv[4][2];
  uint32_t bw[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 32 * wave + 8 * lg + 2 * q + e;
      const int j = c < r ? c : (c < 2 * r ? c - r : 0);
      tv[q][e] = trow[j];
      bw[q][e] = brow[j];
    }
  GvLora o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float av[2];
    uint32_t bv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 32 * wave + 8 * lg + 2 * q + e;
      const bool in = c < 2 * r;
      float hi, lo;
      split_bf16(s * tv[q][e], hi, lo);
      av[e] = !in ? 0.0f : (c < r ? hi : lo);
      bv[e] = in ? bw[q][e] : 0u;
    }
    o.a[q] = pack_bf16x2(av[0], av[1]);
    o.b[q] = bv[0] | (bv[1] << 16);
  }
  return o;
}
__device__ __forceinline__ f32x4_t gv_lora_mfma(const GvLora& l, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(l.a), as_bf16x8(l.b), acc, 0, 0, 0);
}

// Sub-step outer, row group inner: consecutive MFMAs go to different
// accumulators, so none waits for the previous one. The pair lookups of two
// row groups (8 LDS reads) are issued together, ahead of their first use
// (the scheduling barriers keep them there): with the register budget of
// four waves per SIMD the compiler otherwise waits for each lookup before
// issuing the next, exposing the LDS latency once per code byte.
template <int RG>
__device__ __forceinline__ void gv_compute(const GvStage<RG>& st, const f32x2_t* sPair, const float* sC,
                                           int pitch, int li, f32x4_t (&acc)[RG]) {
  constexpr int GB = RG < 2 ? RG : 2;   // row groups per lookup batch
  float cp[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) cp[g] = sC[(16 * g + li) * pitch + st.bl] * st.live;   // c * 0 = 0
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int g0 = 0; g0 < RG; g0 += GB) {
      f32x2_t q[GB][4];
#pragma unroll
      for (int gg = 0; gg < GB; ++gg)
#pragma unroll
        for (int b = 0; b < 4; ++b) q[gg][b] = sPair[(st.code[g0 + gg][u] >> (8 * b)) & 0xFFu];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gg = 0; gg < GB; ++gg) {
        const int g = g0 + gg;
        u32x4_t bv;
#pragma unroll
        for (int b = 0; b < 4; ++b) bv[b] = pack_bf16x2(q[gg][b].x * cp[g], q[gg][b].y * cp[g]);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[u]), as_bf16x8(bv), acc[g], 0, 0, 0);
      }
    }
}

template <int RG, bool DQ, bool OUT_F32, bool TK>
__global__ __launch_bounds__(64 * GV_WAVES, 2) void k_gemv_nf4(GemvParams p) {
  // one LDS object with the pair table first: at LDS address 0 a lookup
  // address is one shift of the code byte
  constexpr int JTK = GV_TR / 16;
  struct __attribute__((aligned(16))) Lds {
    f32x2_t pair[256];
    float c[GV_CTAB];   // constants [16 RG rows][nb + 1]; then partial sums
    f32x4_t tp[TK ? GV_WAVES * JTK * 64 : 1];   // TK: the waves' partial sums of t
    float t[16 * 128];                         // t [tokens][r]
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
  // stages wave, wave + 8, wave + 16, ...: the two stages that share a
  // 128-byte line of a code row (stages 2j and 2j + 1) are read by two waves
  // in the same iteration, so the line is fetched once
  const int nsw = (ns - wave + GV_WAVES - 1) / GV_WAVES;

  const uint8_t* crow[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) crow[g] = p.w.codes + min(n0 + 16 * g + li, N - 1) * (K / 2);   // rows past N: not stored
  const uint16_t* xrow = p.X + min((int64_t)li, p.M - 1) * K;

  // first stage's loads go out before the constant table is built
  GvStage<RG> s0, s1;
  gv_load<RG>(crow, xrow, lg, wave, ns, ns, nb, s0);

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
  if constexpr (TK) {
    // this wave's partial t over its stages: MFMA rows = tokens (X rows li,
    // clamped to M - 1), columns = rows 16 jt + li of A (clamped to r - 1;
    // their sums are not used), the main loop's k layout
    f32x4_t tacc[JTK];
#pragma unroll
    for (int jt = 0; jt < JTK; ++jt) tacc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* arow[JTK];
#pragma unroll
    for (int jt = 0; jt < JTK; ++jt) arow[jt] = p.A + (int64_t)min(16 * jt + li, p.r - 1) * K;
    for (int i = 0; i < nsw; ++i) {
      const int bl = 2 * (wave + GV_WAVES * i) + (lg >> 1);
      const bool live = bl < nb;   // K/64 odd: the last stage's second block is past the row
      const int64_t off = (int64_t)min(bl, nb - 1) * 64 + 32 * (lg & 1);
      u32x4_t xa[4], aa[JTK][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xa[u] = ld16(xrow + off + 8 * u);
#pragma unroll
        for (int jt = 0; jt < JTK; ++jt) aa[jt][u] = ld16(arow[jt] + off + 8 * u);
        if (!live) xa[u] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int jt = 0; jt < JTK; ++jt)
          if (jt == 0 || p.r > 16)   // r <= 16: one column tile
            tacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u]), as_bf16x8(aa[jt][u]), tacc[jt], 0,
                                                               0, 0);
    }
#pragma unroll
    for (int jt = 0; jt < JTK; ++jt) lds.tp[(wave * JTK + jt) * 64 + lane] = tacc[jt];
  } else {
    // t given: staged in LDS for the LoRA step, the sum of its tparts
    // partial sums in part order (stored by workgroup 0 when t_out is set)
    const int64_t nt = p.M * p.r;
    for (int idx = threadIdx.x; idx < nt; idx += 64 * GV_WAVES) {
      float v = p.t[idx];
      for (int k = 1; k < p.tparts; ++k) v += p.t[k * nt + idx];
      lds.t[idx] = v;
      if (blockIdx.x == 0 && p.t_out) p.t_out[idx] = v;
    }
  }
  __syncthreads();
  if constexpr (TK) {
    // t[m][j] = sum over the waves in order; lane (li, lg) of a partial holds
    // tokens 4 lg + v of column li
    for (int idx = threadIdx.x; idx < 16 * p.r; idx += 64 * GV_WAVES) {
      const int m = idx / p.r, j = idx - m * p.r;
      const int ln = (j & 15) + 16 * (m >> 2), v = m & 3;
      float acc_t = 0.0f;
#pragma unroll
      for (int w = 0; w < GV_WAVES; ++w) acc_t += lds.tp[(w * JTK + (j >> 4)) * 64 + ln][v];
      lds.t[idx] = acc_t;
      if (blockIdx.x == 0 && m < p.M && p.t_out) p.t_out[idx] = acc_t;
    }
    __syncthreads();
  }

  // the LoRA operands are loaded only now (held through the table build they
  // would cost registers), all row groups' loads before the first MFMA
  f32x4_t acc[RG];
  if (gv_lora_live(wave, p.r)) {
    GvLora lo[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
      lo[g] = gv_lora_load(lds.t, p.B, p.M, p.r, p.s, wave, li, lg, min(n0 + 16 * g + li, N - 1));
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g] = gv_lora_mfma(lo[g], f32x4_t{0.f, 0.f, 0.f, 0.f});
  } else {
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  __builtin_amdgcn_sched_barrier(0);

  // The scheduling barriers keep each stage's loads where they are issued
  // (left alone, the compiler sinks them next to their first use and the
  // wave then waits for them).
  for (int i = 0; i < nsw; i += 2) {
    gv_load<RG>(crow, xrow, lg, wave + GV_WAVES * (i + 1), ns, ns, nb, s1);
    __builtin_amdgcn_sched_barrier(0);
    gv_compute<RG>(s0, sPair, sC, pitch, li, acc);
    gv_load<RG>(crow, xrow, lg, wave + GV_WAVES * (i + 2), ns, ns, nb, s0);
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
      if (OUT_F32) reinterpret_cast<float*>(p.out)[m * N + n] = h;
      else reinterpret_cast<uint16_t*>(p.out)[m * N + n] = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
    }
  }
}

// ===========================================================================
// Decode GEMV (M <= 16), per-channel codebook weight. The NF4 kernel's tiling
// with one row group per workgroup (16 weight rows, shared by all 8 waves).
// Lane (li, lg) takes codes 32 (lg & 1) + [0, 32) of block 2 ss + (lg >> 1)
// of row n0 + li: bit-plane p of those codes is one 32-bit word, at byte
// 8 b (block) + 8 p + 4 (lg & 1) of the row (b its width), read as 0 for
// p >= b. Two adjacent codes become one MFMA B word through a per-row LDS
// table of level pairs whose index interleaves the two codes' bits (bit 2p:
// bit p of the first code, bit 2p + 1: bit p of the second), so an index is
// the 2-bit fields of the plane words at the pair's position, one field per
// plane. The number of planes handled is the largest width among the
// workgroup's 16 rows (a template parameter chosen per workgroup).
// ===========================================================================
constexpr int CB_TAB = 257;   // level pairs per row: 256 + 1 of padding (rows start on different banks)

size_t cb_gemv_lds_bytes(int64_t K) {
  const size_t rest = std::max<size_t>(16 * (size_t)(K / 64 + 1), (size_t)GV_WAVES * 4 * 64);
  return (size_t)16 * CB_TAB * 8 + 16 * 16 * 4 + rest * 4;
}

struct CbStage {
  uint32_t pl[4];   // bit-planes of the lane's 32 codes (bit j: code j)
  u32x4_t x[4];     // X fragments, k = 32 (lg & 1) + 8 u + [0, 8) of the block
  int bl;
  float live;
};

template <int PB>
__device__ __forceinline__ void cb_load(const uint8_t* rowp, int bw, const uint16_t* xrow, int lg, int st2,
                                        int e1, int ns, int nb, CbStage& st) {
  const int ss = min(st2, ns - 1);
  const int bl = 2 * ss + (lg >> 1);
  st.live = (st2 < e1 && bl < nb) ? 1.0f : 0.0f;
  st.bl = min(bl, nb - 1);
  const uint8_t* src = rowp + (int64_t)st.bl * 8 * bw + 4 * (lg & 1);
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    // planes past the row's width re-read its last plane (in bounds) and drop it
    const uint32_t v = *reinterpret_cast<const uint32_t*>(src + 8 * min(p, bw - 1));
    st.pl[p] = p < bw ? v : 0u;
  }
  const uint16_t* xs = xrow + (int64_t)st.bl * 64 + 32 * (lg & 1);
#pragma unroll
  for (int u = 0; u < 4; ++u) st.x[u] = ld16(xs + 8 * u);
}

template <int PB>
__device__ __forceinline__ void cb_compute(const CbStage& st, const f32x2_t* tab, const float* sC, int pitch,
                                           int li, f32x4_t& acc) {
  const float cp = sC[li * pitch + st.bl] * st.live;   // c * 0 = 0
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f32x2_t q[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int j = 8 * u + 2 * h;
      uint32_t idx = (st.pl[0] >> j) & 3u;
#pragma unroll
      for (int p = 1; p < PB; ++p) idx |= ((st.pl[p] >> j) & 3u) << (2 * p);
      q[h] = tab[idx];
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t bv;
#pragma unroll
    for (int h = 0; h < 4; ++h) bv[h] = pack_bf16x2(q[h].x * cp, q[h].y * cp);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.x[u]), as_bf16x8(bv), acc, 0, 0, 0);
  }
}

template <int PB, bool DQ>
__device__ __forceinline__ f32x4_t cb_body(const GemvParams& p, unsigned char* lds, int64_t n0, const uint8_t* rowp,
                                           int bw, const uint16_t* xrow) {
  f32x2_t* sTab = reinterpret_cast<f32x2_t*>(lds);                  // [16][CB_TAB]
  float* sLv = reinterpret_cast<float*>(lds + 16 * CB_TAB * 8);      // [16][16] levels
  float* sC = sLv + 256;                                              // [16][nb + 1]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t N = p.w.N, K = p.w.K;
  const int nb = (int)(K / 64), pitch = nb + 1;
  const int ns = (int)((K + 127) / 128);
  // stages wave, wave + 8, wave + 16, ...: the two stages that share a
  // 128-byte line of a code row (stages 2j and 2j + 1) are read by two waves
  // in the same iteration, so the line is fetched once
  const int nsw = (ns - wave + GV_WAVES - 1) / GV_WAVES;

  CbStage s0, s1;
  cb_load<PB>(rowp, bw, xrow, lg, wave, ns, ns, nb, s0);   // out before the tables are built
  const bool lora_live = gv_lora_live(wave, p.r);
  GvLora lr{};
  if (lora_live) lr = gv_lora_load(p.t, p.B, p.M, p.r, p.s, wave, li, lg, min(n0 + li, N - 1));

  if (threadIdx.x < 256) sLv[threadIdx.x] = p.w.levels[min(n0 + (threadIdx.x >> 4), N - 1) * 16 + (threadIdx.x & 15)];
  const float mean = DQ ? *p.w.qc.dq_mean : 0.0f;
  const int ncon = 16 * nb;
#pragma unroll 4
  for (int i = threadIdx.x; i < ncon; i += 64 * GV_WAVES) {
    const int rr = i / nb, bl = i - rr * nb;
    const int64_t blk = min(n0 + rr, N - 1) * nb + bl;
    sC[rr * pitch + bl] = DQ ? __builtin_fmaf(e4m3_decode(p.w.qc.absmax_q[blk]), p.w.qc.dq_scale[blk >> 8], mean)
                             : p.w.qc.absmax[blk];
  }
  __syncthreads();
  {
    // 32 threads per row, 8 entries each: entry idx = (first level, second
    // level) with the codes read from the even and the odd bits of idx
    const int rr = threadIdx.x >> 5;
    const float* L = sLv + 16 * rr;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t idx = (threadIdx.x & 31) + 32 * k;
      const uint32_t c0 = (idx & 1u) | ((idx >> 1) & 2u) | ((idx >> 2) & 4u) | ((idx >> 3) & 8u);
      const uint32_t c1 = ((idx >> 1) & 1u) | ((idx >> 2) & 2u) | ((idx >> 3) & 4u) | ((idx >> 4) & 8u);
      sTab[rr * CB_TAB + idx] = f32x2_t{L[c0], L[c1]};
    }
  }
  __syncthreads();

  const f32x2_t* tab = sTab + li * CB_TAB;
  f32x4_t acc = lora_live ? gv_lora_mfma(lr, f32x4_t{0.f, 0.f, 0.f, 0.f}) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nsw; i += 2) {
    cb_load<PB>(rowp, bw, xrow, lg, wave + GV_WAVES * (i + 1), ns, ns, nb, s1);
    __builtin_amdgcn_sched_barrier(0);
    cb_compute<PB>(s0, tab, sC, pitch, li, acc);
    cb_load<PB>(rowp, bw, xrow, lg, wave + GV_WAVES * (i + 2), ns, ns, nb, s0);
    __builtin_amdgcn_sched_barrier(0);
    cb_compute<PB>(s1, tab, sC, pitch, li, acc);
  }
  return acc;
}

template <bool DQ, bool OUT_F32>
__global__ __launch_bounds__(64 * GV_WAVES, 2) void k_gemv_codebook(GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char cb_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int64_t N = p.w.N, K = p.w.K;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t row = min(n0 + li, N - 1);   // rows past N: not stored
  const int bw = min(max((int)p.w.row_bits[row], 1), 4);
  const uint8_t* rowp = p.w.codes + p.w.row_offset[row];
  const uint16_t* xrow = p.X + min((int64_t)li, p.M - 1) * K;
  const int pb = (int)row16_max((float)bw);   // the 16 rows' widest, the same in every wave

  f32x4_t acc;
  switch (pb) {
    case 1: acc = cb_body<1, DQ>(p, cb_lds, n0, rowp, bw, xrow); break;
    case 2: acc = cb_body<2, DQ>(p, cb_lds, n0, rowp, bw, xrow); break;
    case 3: acc = cb_body<3, DQ>(p, cb_lds, n0, rowp, bw, xrow); break;
    default: acc = cb_body<4, DQ>(p, cb_lds, n0, rowp, bw, xrow); break;
  }

  // reduce the 8 K-splits in the constant region (free now)
  __syncthreads();
  float* sR = reinterpret_cast<float*>(cb_lds + 16 * CB_TAB * 8) + 256;   // [wave][v][lane]
#pragma unroll
  for (int v = 0; v < 4; ++v) sR[(wave * 4 + v) * 64 + lane] = acc[v];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int ln = threadIdx.x;
    const int64_t n = n0 + (ln & 15);
    if (n < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = 4 * (ln >> 4) + v;
        if (m >= p.M) continue;
        float h = 0.0f;
#pragma unroll
        for (int w = 0; w < GV_WAVES; ++w) h += sR[(w * 4 + v) * 64 + ln];
        if (OUT_F32) reinterpret_cast<float*>(p.out)[m * N + n] = h;
        else reinterpret_cast<uint16_t*>(p.out)[m * N + n] = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
      }
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
// needed.
// With RT > 0 the second operand is given transposed, Rt [C, r] (B for
// u = G B; RT = 1: r % 8 == 0, rows read in 16-byte pieces; RT = 2: any r):
// per 64-column block and 16 rows j, lane l loads row 64 bk + l of Rt (16
// values) and writes it as column l of a 16 x 64 tile in the wave's own LDS
// area, from which the fragments are read as above (no barrier: only the
// wave itself touches the area, and its LDS operations run in order).
constexpr int RS_TP = 72;   // bf16 per row of the transposed tile (144 bytes)

template <int JT, int W, int RT, int UB>
__global__ __launch_bounds__(64 * W) void k_row_skinny(const uint16_t* __restrict__ Q, int64_t M, int64_t C,
                                                       const uint16_t* __restrict__ R, int r,
                                                       float* __restrict__ out) {
  constexpr int kPart = W * JT * 64 * 16, kTile = RT ? W * 16 * RS_TP * 2 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char sRaw[kPart > kTile ? kPart : kTile];
  f32x4_t (*sPart)[JT][64] = reinterpret_cast<f32x4_t (*)[JT][64]>(sRaw);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* sT = reinterpret_cast<uint16_t*>(sRaw) + wave * 16 * RS_TP;   // RT: this wave's 16 x 64 tile
  const int li = lane & 15, lg = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const uint16_t* qrow = Q + min(row0 + li, M - 1) * C + 16 * lg;   // rows past M: not stored
  const uint16_t* rrow[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) rrow[jt] = RT ? R : R + (int64_t)min(16 * jt + li, r - 1) * C + 16 * lg;
  // column part blockIdx.y of gridDim.y: a contiguous range of 64-column
  // blocks, its partial sums stored at out + part * M * r
  const int64_t blocks = (C + 63) / 64;
  const int64_t bpp = (blocks + gridDim.y - 1) / gridDim.y;
  const int64_t p_begin = min(blocks, (int64_t)blockIdx.y * bpp), p_end = min(blocks, p_begin + bpp);
  const int64_t per = (p_end - p_begin + W - 1) / W;
  const int64_t b_begin = min(p_end, p_begin + wave * per), b_end = min(p_end, b_begin + per);
  out += (int64_t)blockIdx.y * M * r;
  f32x4_t acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr bool PIPE = RT == 0 && JT >= 3;
  if constexpr (PIPE) {
    // r > 32: two register sets of one block each, the loads of the next in
    // flight while the current one is multiplied (blocks, then halves, then
    // row tiles: the same accumulation order as one set at a time). At
    // r = 64 over 11008 columns 65.0 -> 59.1 us; at r <= 32 the single set
    // of up to four blocks below was faster.
    constexpr int U = 1;
    auto load = [&](int64_t bk, u32x4_t (&a)[U][2], u32x4_t (&b)[U][2][JT]) {
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
    };
    auto mma = [&](const u32x4_t (&a)[U][2], const u32x4_t (&b)[U][2][JT]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int jt = 0; jt < JT; ++jt)
            acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][h]), as_bf16x8(b[u][h][jt]), acc[jt],
                                                              0, 0, 0);
    };
    u32x4_t a0[U][2], b0[U][2][JT], a1[U][2], b1[U][2][JT];
    if (b_begin < b_end) load(b_begin, a0, b0);
    for (int64_t bk = b_begin; bk < b_end; bk += 2 * U) {
      if (bk + U < b_end) load(bk + U, a1, b1);
      mma(a0, b0);
      if (bk + U >= b_end) break;
      if (bk + 2 * U < b_end) load(bk + 2 * U, a0, b0);
      mma(a1, b1);
    }
  }
  // UB 64-column blocks with loads in flight together (every lane issues the
  // loads of all UB blocks, live or not, and the time follows that count:
  // the launcher sizes UB to the blocks a wave has)
  constexpr int U = PIPE ? 1 : UB;
  for (int64_t bk = b_begin; !PIPE && bk < b_end; bk += U) {
    u32x4_t a[U][2], b[U][2][JT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t cc = 64 * (bk + u) + 8 * h;   // + 16 lg in the row pointers
        const bool ok = bk + u < b_end && cc + 16 * lg + 8 <= C;
        const int64_t off = ok ? cc : -16 * lg;     // a lane past the end reads columns 0..7 and adds 0
        a[u][h] = ld16(qrow + off);
        if constexpr (!RT) {
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) b[u][h][jt] = ld16(rrow[jt] + off);
        }
        if (!ok) zero(a[u][h]);
      }
    if constexpr (RT) {
      // rows 64 (bk + u) + lane of Rt, 16 values per jt (zero past C or r)
      u32x4_t t[U][JT][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = 64 * (bk + u) + lane;
        const bool live = bk + u < b_end && c < C;
        const uint16_t* src = R + (live ? c : 0) * r;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int j0 = 16 * jt + 8 * q;
            if constexpr (RT == 1) {
              if (live && j0 < r) t[u][jt][q] = ld16(src + j0);
              else zero(t[u][jt][q]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t lo = (live && j0 + 2 * e < r) ? src[j0 + 2 * e] : 0u;
                const uint32_t hi = (live && j0 + 2 * e + 1 < r) ? src[j0 + 2 * e + 1] : 0u;
                t[u][jt][q][e] = lo | (hi << 16);
              }
            }
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              sT[(8 * q + e) * RS_TP + lane] = (uint16_t)(t[u][jt][q][e >> 1] >> (16 * (e & 1)));
#pragma unroll
          for (int h = 0; h < 2; ++h) b[u][h][jt] = ld16(sT + li * RS_TP + 16 * lg + 8 * h);
        }
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
  if constexpr (RT) __syncthreads();   // the partial sums reuse the tiles' LDS
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
// [M, r] small, Q bfloat16 [M, C] streamed once. Per 32 rows of m, P is split
// into [hi(P)^T ; lo(P)^T] (bfloat16 [2r][32]; hi + lo carries P to about
// 2^-17) in LDS, so an MFMA A fragment is one 16-byte LDS read. The Q tile
// [32 m x 128 c] goes through LDS too and is gathered along m for the B
// fragments. Both are loaded one chunk ahead. Workgroup: 128 columns x one m-split, wave: 32 columns, MFMA
// 32x32x16 over the 2r product rows; hi and lo rows are added in registers
// when r % 32 == 0 or r == 16 (partner row in the same lane), otherwise both
// are kept. Each workgroup writes the partial sums of its m-split;
// k_reduce_splits2 adds them.
// One job of the column form: product pt2^T-by-Q over its m-splits, in
// `tiles` column tiles of 128.
struct ColJob {
  const float* P;
  const uint16_t* Q;
  int64_t C;
  int64_t m_per_split;
  int splits;
  unsigned tiles;
  float* part;
};

// Two jobs share one launch (same M and r): workgroups x < j0.tiles take
// job 0, the rest job 1; split rows y past a job's own split count exit.
constexpr int CS_PP = 40;   // bf16 per LDS row of the split P tile (80 bytes)

template <int JT2>
__global__ __launch_bounds__(256) void k_col_skinny(ColJob j0, ColJob j1, int64_t M, int r, int combine) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[32 * (128 + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sP[32 * JT2 * CS_PP];
  const bool second = blockIdx.x >= j0.tiles;
  const ColJob jb = second ? j1 : j0;
  if ((int)blockIdx.y >= jb.splits) return;   // the whole workgroup
  const float* __restrict__ P = jb.P;
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
  // A-fragment rows of the split tile (rows past 2r read row 0: their
  // products are not used)
  const uint16_t* arow[JT2];
#pragma unroll
  for (int jt = 0; jt < JT2; ++jt) {
    const int j = 32 * jt + li;
    arow[jt] = sP + (j < rows2 ? j : 0) * CS_PP + 8 * lh;
  }
  // The 32 r values of P for one chunk of 32 rows: thread t takes elements
  // t + 256 q (q < 2 JT2 covers 32 r since r <= 16 JT2); the next chunk's
  // loads are issued before the current chunk's products.
  constexpr int PQ = 2 * JT2;
  float pv[PQ];
  auto load_p = [&](int64_t mb) {
#pragma unroll
    for (int q = 0; q < PQ; ++q) {
      const int idx = threadIdx.x + 256 * q;
      const int row = idx / r;
      const int64_t m = mb + row;
      pv[q] = (idx < 32 * r && m < m_end) ? P[m * r + (idx - row * r)] : 0.0f;
    }
  };
  // the Q tile of a chunk: thread t takes 16-byte pieces t and t + 256 of the
  // 32 x 128 tile (zero past m_end and C), loaded one chunk ahead as well
  u32x4_t qv[2];
  auto load_q = [&](int64_t mb) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = threadIdx.x + 256 * q;
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
      qv[q] = v;
    }
  };
  load_p(m_begin);
  load_q(m_begin);
  for (int64_t mb = m_begin; mb < m_end; mb += 32) {
    // sP[j][m - mb] = hi(P[m][j]), sP[j + r][m - mb] = lo(P[m][j]); zero past m_end
#pragma unroll
    for (int q = 0; q < PQ; ++q) {
      const int idx = threadIdx.x + 256 * q;
      if (idx < 32 * r) {
        const int row = idx / r, j = idx - row * r;
        float hi, lo;
        split_bf16(pv[q], hi, lo);
        sP[j * CS_PP + row] = (uint16_t)(pack_bf16x2(hi, 0.f) & 0xFFFFu);
        sP[(j + r) * CS_PP + row] = (uint16_t)(pack_bf16x2(lo, 0.f) & 0xFFFFu);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = threadIdx.x + 256 * q;
      *reinterpret_cast<u32x4_t*>(sQ + (idx / 16) * (128 + 8) + (idx % 16) * 8) = qv[q];
    }
    load_p(mb + 32);
    load_q(mb + 32);
    __syncthreads();
    u32x4_t af[2][JT2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int jt = 0; jt < JT2; ++jt) af[s][jt] = ld16(arow[jt] + 16 * s);
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

// A workgroup's time follows the load instructions its waves issue (about
// 3 us + 0.4 us per 16 loads of a wave, the waves' loads taking turns), so
// the columns are split into parts while the row groups leave CUs idle: at
// 2048 rows (128 row groups) and 4096 columns two parts take 5.8 instead of
// 9.4 us. Each part keeps at least one 64-column block per wave; at most 4.
int row_skinny_parts(int64_t M, int64_t C) {
  const int64_t groups = (M + 15) / 16, blocks = (C + 63) / 64;
  int P = 1;
  while (P < 4 && groups * 2 * P <= 8 * kCusPerXcd && blocks / (2 * P) >= 16) P *= 2;
  return P;
}

// Blocks in flight per wave: as many as a wave has (1, 2 or 4; more take
// further rounds).
static int row_skinny_ub(int64_t C, int parts, int W) {
  const int64_t blocks = (C + 63) / 64, bpp = (blocks + parts - 1) / parts, per = (bpp + W - 1) / W;
  return per <= 1 ? 1 : (per <= 2 ? 2 : 4);
}

hipError_t launch_row_skinny(const uint16_t* Q, int64_t M, int64_t C, const uint16_t* R, int r, float* out,
                             hipStream_t s, int parts) {
  if (parts < 1 || parts > 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + 15) / 16), (unsigned)parts);
  const int jt = (r + 15) / 16;
  if (jt <= 2) {
    const int ub = row_skinny_ub(C, parts, 16);
#define LQ_RS(JT, UB) hipLaunchKernelGGL((k_row_skinny<JT, 16, 0, UB>), grid, dim3(1024), 0, s, Q, M, C, R, r, out)
    if (jt == 1) {
      if (ub == 1) LQ_RS(1, 1);
      else if (ub == 2) LQ_RS(1, 2);
      else LQ_RS(1, 4);
    } else {
      if (ub == 1) LQ_RS(2, 1);
      else if (ub == 2) LQ_RS(2, 2);
      else LQ_RS(2, 4);
    }
#undef LQ_RS
    return hipGetLastError();
  }
  switch (jt) {
#define LQ_RS(JT) case JT: hipLaunchKernelGGL((k_row_skinny<JT, 8, 0, 1>), grid, dim3(512), 0, s, Q, M, C, R, r, out); break;
    LQ_RS(3) LQ_RS(4) LQ_RS(5) LQ_RS(6) LQ_RS(7) LQ_RS(8)
#undef LQ_RS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Each workgroup transposes the whole of Rt for its 16 rows, so this form
// pays only while that is small: r <= 16 (at r = 64 over 11008 columns it
// cost more than a separate transpose launch).
hipError_t launch_row_skinny_rt(const uint16_t* Q, int64_t M, int64_t C, const uint16_t* Rt, int r, float* out,
                                hipStream_t s, int parts) {
  if (r > 16 || parts < 1 || parts > 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + 15) / 16), (unsigned)parts);
  const int ub = row_skinny_ub(C, parts, 16);
#define LQ_RS(RT, UB) hipLaunchKernelGGL((k_row_skinny<1, 16, RT, UB>), grid, dim3(1024), 0, s, Q, M, C, Rt, r, out)
  if (r % 8 == 0) {
    if (ub == 1) LQ_RS(1, 1);
    else if (ub == 2) LQ_RS(1, 2);
    else LQ_RS(1, 4);
  } else {
    if (ub == 1) LQ_RS(2, 1);
    else if (ub == 2) LQ_RS(2, 2);
    else LQ_RS(2, 4);
  }
#undef LQ_RS
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
    job[njobs] = ColJob{q.P, q.Q, q.C, m_per_split, real_splits, (unsigned)((q.C + 127) / 128), q.ws};
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
#define LQ_CS(JT) case JT: hipLaunchKernelGGL(k_col_skinny<JT>, grid, dim3(256), 0, s, job[0], job[1], M, r, combine); break;
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

// The GEMM's schedule on MI355X (256 CUs in 8 XCDs of 32, kCusPerXcd), one
// workgroup per CU. Tiles are split only when each XCD has at least one full
// round and the contraction has at least 16 steps.
static int split_cpx(int64_t M, int64_t Ncols, int64_t Kc) {
  return (Kc + BK - 1) / BK >= 16 ? kCusPerXcd : 0;
}
static int64_t split_tiles(int64_t M, int64_t Ncols, int64_t Kc) {
  const int cpx = split_cpx(M, Ncols, Kc);
  const int64_t total = ((M + BM - 1) / BM) * ((Ncols + BN - 1) / BN);
  int64_t n = 0;
  for (int x = 0; x < 8; ++x) n += xcd_splits(xcd_tiles(total, x), cpx);
  return n;
}
static int64_t gemm_grid(int64_t M, int64_t Ncols, int64_t Kc) {
  const int cpx = split_cpx(M, Ncols, Kc);
  const int64_t total = ((M + BM - 1) / BM) * ((Ncols + BN - 1) / BN);
  int64_t longest = 0;
  for (int x = 0; x < 8; ++x) {
    const int64_t n_x = xcd_tiles(total, x);
    longest = std::max(longest, n_x + xcd_splits(n_x, cpx));
  }
  return 8 * longest;
}
static size_t split_part_bytes(int64_t M, int64_t Ncols, int64_t Kc) {
  return align256((size_t)split_tiles(M, Ncols, Kc) * 2 * BM * BN * sizeof(float));
}

// Workspace of the forward / backward GEMM: (codebook format) the dequantized
// bf16 weight, then the split tiles' partial sums (when the schedule splits).
size_t gemm_ws_bytes(const QWeight& w, int64_t M, int, bool fwd) {
  const size_t wbf = w.format == LQ_FMT_CODEBOOK ? align256((size_t)w.N * w.K * sizeof(uint16_t)) : 0;
  return wbf + (fwd ? split_part_bytes(M, w.N, w.K) : split_part_bytes(M, w.K, w.N));
}

// Adds the split tiles' halves (a second launch, only when the schedule splits).
template <bool OUT_F32>
static hipError_t launch_split_fixup(const GemmParams& p, hipStream_t st) {
  const int64_t n = split_tiles(p.M, p.Ncols, p.Kc);
  if (n == 0) return hipSuccess;
  const int64_t threads = n * (BM * BN / 4);
  hipLaunchKernelGGL(k_split_fixup<OUT_F32>, dim3((unsigned)std::min<int64_t>((threads + 255) / 256, 4096)),
                     dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// The LoRA segment's sources (read by the GEMM itself).
static void set_lora(GemmParams& p, const float* L, const uint16_t* lb, int r, float s, bool fwd) {
  p.L = L;
  p.lb = lb;
  p.r = r;
  p.s = s;
  p.fwd = fwd ? 1 : 0;
  p.R2 = lora_seg_cols(r);
  p.lvec = (r % 8 == 0 && reinterpret_cast<uintptr_t>(L) % 16 == 0) ? 1 : 0;
}

static GemmParams make_params(const QWeight& w, const uint16_t* A, int64_t M, int64_t Ncols, int64_t Kc,
                              void* out) {
  GemmParams p;
  p.A = A; p.M = M; p.Ncols = Ncols; p.Kc = Kc; p.out = out;
  p.L = nullptr; p.lb = nullptr; p.r = 0; p.s = 0.0f; p.fwd = 1; p.R2 = 0; p.lvec = 0;
  // 32 workgroups are resident per XCD: 2 A row-tiles x 16 weight tiles
  // minimise the bytes they pull into the XCD's L2.
  p.gm = (int)std::min<int64_t>(2, (M + BM - 1) / BM);
  p.w = w;
  p.lv = tables().lv;
  p.wbf = nullptr;
  p.red[0] = p.red[1] = SplitJob{nullptr, 0, 0, 0, 0, 0, 0.0f, nullptr, 0};
  p.red_n[0] = p.red_n[1] = 0;
  p.cpx = split_cpx(M, Ncols, Kc);
  p.part = nullptr;
  return p;
}

hipError_t launch_gemm_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype, uint16_t* ws,
                           hipStream_t st) {
  GemmParams p = make_params(w, X, M, w.N, w.K, H);
  set_lora(p, t, B, r, s, true);
  hipError_t e = hipSuccess;
  const int64_t tiles = gemm_grid(M, w.N, w.K);
  LQ_DASSERT(M > 0 && w.K % 64 == 0 && tiles > 0 && tiles < (int64_t(1) << 31));
  LQ_DASSERT(r >= 1 && r <= 128 && p.R2 % BK == 0);
  const dim3 grid((unsigned)tiles);
  const size_t wbf_bytes = w.format == LQ_FMT_CODEBOOK ? align256((size_t)w.N * w.K * sizeof(uint16_t)) : 0;
  p.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + wbf_bytes);   // used only by split tiles
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
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return f32 ? launch_split_fixup<true>(p, st) : launch_split_fixup<false>(p, st);
}

hipError_t launch_gemm_bwd(const QWeight& w, const uint16_t* G, int64_t M, const float* u,
                           const uint16_t* A, int r, float s, uint16_t* gX, uint16_t* ws, hipStream_t st,
                           const SplitJobDesc* red_a, const SplitJobDesc* red_b) {
  GemmParams p = make_params(w, G, M, w.K, w.N, gX);
  set_lora(p, u, A, r, s, false);
  const SplitJobDesc* rd[2] = {red_a, red_b};
  for (int i = 0; i < 2; ++i) {
    if (!rd[i] || !rd[i]->out) continue;
    p.red[i] = SplitJob{rd[i]->part, rd[i]->splits, rd[i]->rows, rd[i]->cols, rd[i]->srows, rd[i]->pair,
                        rd[i]->scale, rd[i]->out, rd[i]->transposed};
    p.red_n[i] = rd[i]->rows * rd[i]->cols;
  }
  hipError_t e = hipSuccess;
  const int64_t tiles = gemm_grid(M, w.K, w.N);
  LQ_DASSERT(M > 0 && w.N % 8 == 0 && w.K % 64 == 0 && tiles > 0 && tiles < (int64_t(1) << 31));
  LQ_DASSERT(r >= 1 && r <= 128 && p.R2 % BK == 0);
  const dim3 grid((unsigned)tiles);
  const size_t wbf_bytes = w.format == LQ_FMT_CODEBOOK ? align256((size_t)w.N * w.K * sizeof(uint16_t)) : 0;
  p.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + wbf_bytes);   // used only by split tiles
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
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_split_fixup<false>(p, st);
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

// Codebook weights: while the kernel's LDS (pair tables, levels, constants)
// stays within 64 KB, i.e. K <= 32576.
bool gemv_supported(const QWeight& w) {
  if (w.format == LQ_FMT_CODEBOOK) return cb_gemv_lds_bytes(w.K) <= 65536;
  return w.format == LQ_FMT_NF4 && gemv_rg(w.N, w.K, 1) > 0;
}

// Every workgroup that forms t reads all of X and A (from L2) for it. That
// pays while the grid is at most one workgroup per CU (measured: 17.5 ->
// 12.3 us at 1024 x 1024, 19.9 -> 16.9 at 4096 x 4096 and 51.5 -> 46.9 at
// N = 4096, K = 14336, 16 tokens) and costs once CUs hold two (8192 x 8192,
// one token: 23.6 -> 33.3 us; 28672 x 8192: 46.1 -> 54.8).
constexpr int64_t GV_TK_MAX_WGS = 8 * kCusPerXcd;

bool gemv_forms_t(const QWeight& w, int64_t M, int r) {
  if (w.format != LQ_FMT_NF4 || r > GV_TR || M < 1 || M > 16 || !gemv_supported(w)) return false;
  const int rg = gemv_rg(w.N, w.K, M);
  return (w.N + 16 * rg - 1) / (16 * rg) <= GV_TK_MAX_WGS;
}

template <int RG, bool TK>
static void launch_gemv_rg(const GemvParams& p, bool dq, bool f32, hipStream_t st) {
  const dim3 grid((unsigned)((p.w.N + 16 * RG - 1) / (16 * RG))), block(64 * GV_WAVES);
  if (dq && f32) hipLaunchKernelGGL((k_gemv_nf4<RG, true, true, TK>), grid, block, 0, st, p);
  else if (dq) hipLaunchKernelGGL((k_gemv_nf4<RG, true, false, TK>), grid, block, 0, st, p);
  else if (f32) hipLaunchKernelGGL((k_gemv_nf4<RG, false, true, TK>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((k_gemv_nf4<RG, false, false, TK>), grid, block, 0, st, p);
}

hipError_t launch_gemv_fwd(const QWeight& w, const uint16_t* X, int64_t M, const float* t,
                           const uint16_t* B, int r, float s, void* H, int h_dtype,
                           hipStream_t st, const uint16_t* A, float* t_out, int t_parts) {
  if (!gemv_supported(w)) return hipErrorInvalidValue;
  GemvParams p;
  p.X = X; p.M = M; p.t = t; p.B = B; p.r = r; p.s = s; p.out = H; p.w = w; p.lv = tables().lv;
  const bool tk = t == nullptr;   // form t = X A^T in the kernel (NF4, r <= GV_TR)
  p.tparts = tk ? 1 : t_parts;
  p.A = A;
  p.t_out = (tk || t_parts > 1) ? t_out : nullptr;
  if (tk && (w.format != LQ_FMT_NF4 || !A || r > GV_TR)) return hipErrorInvalidValue;
  const bool dq = w.qc.absmax == nullptr, f32 = h_dtype == LQ_F32;
  if (w.format == LQ_FMT_CODEBOOK) {
    if (p.tparts != 1) return hipErrorInvalidValue;   // the codebook kernel reads t as given
    const size_t lds = cb_gemv_lds_bytes(w.K);
    const dim3 grid((unsigned)((w.N + 15) / 16)), block(64 * GV_WAVES);
    LQ_DASSERT(M >= 1 && M <= 16 && w.K % 64 == 0 && lds <= 65536);
    if (dq && f32) hipLaunchKernelGGL((k_gemv_codebook<true, true>), grid, block, lds, st, p);
    else if (dq) hipLaunchKernelGGL((k_gemv_codebook<true, false>), grid, block, lds, st, p);
    else if (f32) hipLaunchKernelGGL((k_gemv_codebook<false, true>), grid, block, lds, st, p);
    else hipLaunchKernelGGL((k_gemv_codebook<false, false>), grid, block, lds, st, p);
    return hipGetLastError();
  }
  const int rg = gemv_rg(w.N, w.K, M);
  LQ_DASSERT(M >= 1 && M <= 16 && w.K % 64 == 0 && (int64_t)16 * rg * (w.K / 64 + 1) <= GV_CTAB);
  if (tk) {
    if (rg == 4) launch_gemv_rg<4, true>(p, dq, f32, st);
    else if (rg == 2) launch_gemv_rg<2, true>(p, dq, f32, st);
    else launch_gemv_rg<1, true>(p, dq, f32, st);
  } else {
    if (rg == 4) launch_gemv_rg<4, false>(p, dq, f32, st);
    else if (rg == 2) launch_gemv_rg<2, false>(p, dq, f32, st);
    else launch_gemv_rg<1, false>(p, dq, f32, st);
  }
  return hipGetLastError();
}

}  // namespace lq
