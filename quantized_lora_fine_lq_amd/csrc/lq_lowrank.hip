// Low-rank initialisation of the adapter (LowRA, sections 3 and 5: the
// quantization error is turned into the starting adapter by LoftQ, five
// alternating steps of quantizing W - B A and a rank-r SVD of the residual).
//
// Kernels:
//   * W - B A with the rank-r product summed in float64 in order of j;
//   * R = W - W' (W' the layer's bf16 weight);
//   * the rank-r SVD of R by randomized subspace iteration: Y = R Omega, then
//     power steps Y = R (R^T Y), each new Y orthonormalised by CholQR2
//     (float64 Gram, Cholesky and the inverse of its factor in one workgroup,
//     then a right multiply); a final Rayleigh-Ritz step takes the
//     eigenvectors of the l x l Gram of R^T Y by cyclic Jacobi in float64 in
//     one workgroup;
//   * ||R - B A||_F^2 with a fixed-order float64 reduction.
// Tall-skinny products keep R row-major and stream it once per product.
#include <algorithm>
#include <cmath>

#include "lq_device.h"

namespace lq {
namespace {

constexpr int LR_MAXL = 96;    // l = r + oversampling, one Jacobi workgroup holds two l x l float64 matrices

// ---- out = float32(W - sum_j B[n][j] A[j][k]), float64 sum in order of j ----
__global__ __launch_bounds__(256) void k_lowrank_sub(const float* __restrict__ W, int64_t N, int64_t K,
                                                     const float* __restrict__ B, const float* __restrict__ A,
                                                     int r, float* __restrict__ out) {
  const int64_t quads = N * K / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (int64_t)gridDim.x * 256) {
    const int64_t e = 4 * i;
    const int64_t n = e / K, k = e - n * K;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int j = 0; j < r; ++j) {
      const double b = (double)B[n * r + j];
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(A + (int64_t)j * K + k);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += b * (double)a[q];   // products exact in float64
    }
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(W + e);
    f32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (float)((double)w[q] - acc[q]);
    *reinterpret_cast<f32x4_t*>(out + e) = o;
  }
}

// ---- R = W - W' (one float32 subtraction) ---------------------------------
__global__ __launch_bounds__(256) void k_residual(const float* __restrict__ W, const uint16_t* __restrict__ Wd,
                                                  int64_t n, float* __restrict__ R) {
  const int64_t quads = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (int64_t)gridDim.x * 256) {
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(W + 4 * i);
    const uint2 d = *reinterpret_cast<const uint2*>(Wd + 4 * i);
    f32x4_t o;
    o[0] = w[0] - bf16lo_to_f32(d.x);
    o[1] = w[1] - bf16hi_to_f32(d.x);
    o[2] = w[2] - bf16lo_to_f32(d.y);
    o[3] = w[3] - bf16hi_to_f32(d.y);
    *reinterpret_cast<f32x4_t*>(R + 4 * i) = o;
  }
}

// ---- tall-skinny products, split over the contraction -----------------------
// TRANS = false: Y[M, l] = X[M, C] V[C, l]   (contraction over C)
// TRANS = true:  Z[C, l] = X[M, C]^T V[M, l] (contraction over M)
// X row-major [M, C] with C % 4 == 0. Workgroup: 128 output rows x all l
// columns over one slice of the contraction (partials [slices, rows_out, l]).
// Tiles are k-major in LDS (32 x 128 of X, 32 x LP of V, LP = l rounded up
// to 32); thread t computes rows 4 (t % 32) .. +3 and TN = LP / 8 columns
// TN (t / 32) .. +TN - 1, reading both operands as 16-byte LDS words.
template <bool TRANS, int TN>
__global__ __launch_bounds__(256) void k_skinny_gemm(const float* __restrict__ X, int64_t M, int64_t C,
                                                     const float* __restrict__ V, int l, int64_t kslice,
                                                     float* __restrict__ part) {
  constexpr int BM = 128, BK = 32, LP = 8 * TN;
  __shared__ __attribute__((aligned(16))) float sA[BK][BM + 4];
  __shared__ __attribute__((aligned(16))) float sV[BK][LP + 4];
  const int t = threadIdx.x;
  const int64_t rows_out = TRANS ? C : M, kc = TRANS ? M : C;
  const int64_t o0 = (int64_t)blockIdx.x * BM;
  const int64_t kb = (int64_t)blockIdx.y * kslice, ke = std::min<int64_t>(kc, kb + kslice);
  const int rg = t & 31, cg = t >> 5;
  float acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;
  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
    if (!TRANS) {
      // rows o0 + t/2, contraction k0 + 16 (t % 2) .. +15, stored transposed
      const int o = t >> 1, kq = (t & 1) * 16;
      const int64_t row = o0 + o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + kq + 4 * q;
        f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (row < M && k + 4 <= ke) v = *reinterpret_cast<const f32x4_t*>(X + row * C + k);
        else if (row < M)
          for (int e = 0; e < 4; ++e) v[e] = (k + e < ke) ? X[row * C + k + e] : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sA[kq + 4 * q + e][o] = v[e];
      }
    } else {
      // contraction rows k0 + t/8, output columns o0 + 16 (t % 8) .. +15
      const int kk = t >> 3, oq = (t & 7) * 16;
      const int64_t krow = k0 + kk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t o = o0 + oq + 4 * q;
        f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (krow < ke && o + 4 <= C) v = *reinterpret_cast<const f32x4_t*>(X + krow * C + o);
        else if (krow < ke)
          for (int e = 0; e < 4; ++e) v[e] = (o + e < C) ? X[krow * C + o + e] : 0.0f;
        *reinterpret_cast<f32x4_t*>(&sA[kk][oq + 4 * q]) = v;
      }
    }
    for (int i = t; i < BK * LP; i += 256) {
      const int kk = i / LP, c = i % LP;   // LP is a compile-time constant
      const int64_t k = k0 + kk;
      sV[kk][c] = (k < ke && c < l) ? V[k * l + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < BK; ++kk) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sA[kk][4 * rg]);
      float v[TN];
#pragma unroll
      for (int j4 = 0; j4 < TN / 4; ++j4) {
        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(&sV[kk][TN * cg + 4 * j4]);
        v[4 * j4] = w[0]; v[4 * j4 + 1] = w[1]; v[4 * j4 + 2] = w[2]; v[4 * j4 + 3] = w[3];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], v[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* dst = part + (int64_t)blockIdx.y * rows_out * l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t o = o0 + 4 * rg + i;
    if (o >= rows_out) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c = TN * cg + j;
      if (c < l) dst[o * l + c] = acc[i][j];
    }
  }
}

// out[i] = sum_s part[s][i] in order of s
__global__ __launch_bounds__(256) void k_sum_splits(const float* __restrict__ part, int splits, int64_t n,
                                                    float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) v += part[(int64_t)s * n + i];
    out[i] = v;
  }
}

// ---- Gram G = Y^T Y in float64: per-workgroup partials, fixed-order sum -----
__global__ __launch_bounds__(256) void k_gram_partial(const float* __restrict__ Y, int64_t M, int l,
                                                      int64_t rows_per_wg, double* __restrict__ part) {
  __shared__ float sY[32][LR_MAXL];
  const int t = threadIdx.x;
  const int64_t mb = (int64_t)blockIdx.x * rows_per_wg, me = std::min<int64_t>(M, mb + rows_per_wg);
  constexpr int PER = (LR_MAXL * LR_MAXL + 255) / 256;
  double acc[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) acc[q] = 0.0;
  const int ll = l * l;
  for (int64_t m0 = mb; m0 < me; m0 += 32) {
    for (int i = t; i < 32 * l; i += 256) {
      const int rr = i / l, cc = i - rr * l;
      const int64_t m = m0 + rr;
      sY[rr][cc] = (m < me) ? Y[m * l + cc] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + 256 * q;
      if (e < ll) {
        const int i = e / l, j = e - i * l;
        double a = acc[q];
        for (int rr = 0; rr < 32; ++rr) a += (double)sY[rr][i] * (double)sY[rr][j];
        acc[q] = a;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = t + 256 * q;
    if (e < ll) part[(int64_t)blockIdx.x * ll + e] = acc[q];
  }
}

__global__ __launch_bounds__(256) void k_gram_finish(const double* __restrict__ part, int parts, int ll,
                                                     double* __restrict__ G) {
  for (int e = blockIdx.x * 256 + threadIdx.x; e < ll; e += gridDim.x * 256) {
    double v = 0.0;
    for (int s0 = 0; s0 < parts; s0 += 16) {   // 16 loads in flight, summed in order
      double x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = (s0 + u < parts) ? part[(int64_t)(s0 + u) * ll + e] : 0.0;
#pragma unroll
      for (int u = 0; u < 16; ++u) v += x[u];
    }
    G[e] = v;
  }
}

// ---- small dense float64 kernels on LDS matrices (one 256-thread workgroup) ---
// Matrices are [D][D + 1] arrays (padded rows); every thread calls each
// routine, which ends with a barrier.

// Cholesky: sL = L with A = L L^T from the lower triangle of sA (destroyed).
// Column step j: every thread forms the pivot d = A[j][j] itself; the
// trailing update uses the unscaled column, A[i][k] -= A[i][j] A[k][j] / d,
// and L's column j goes to sL, so one barrier per step suffices. A pivot at
// or below tol marks a column that depends on the earlier ones: its column
// of L is zero.
template <int D>
__device__ void lds_cholesky(double (*sA)[D + 1], double (*sL)[D + 1], int l, double tol) {
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  for (int i = ty; i < l; i += 16)
    for (int k = tx; k < l; k += 16) sL[i][k] = 0.0;
  __syncthreads();
  for (int j = 0; j < l; ++j) {
    const double d = sA[j][j];
    const bool ok = d > tol && d > 0.0;
    const double piv = ok ? sqrt(d) : 0.0;
    const double inv_d = ok ? 1.0 / d : 0.0;
    if (ty == 0)
      for (int i = j + tx; i < l; i += 16) sL[i][j] = ok ? ((i == j) ? piv : sA[i][j] / piv) : 0.0;
    for (int i = j + 1 + ty; i < l; i += 16) {
      const double aij = sA[i][j] * inv_d;
      for (int k = j + 1 + tx; k <= i; k += 16) sA[i][k] -= aij * sA[k][j];
    }
    __syncthreads();
  }
}

// sI = L^{-1} (lower triangular; a zero pivot gives a zero row) by forward
// substitution one row at a time, each column's dot product split over the
// 16 threads of a row group and reduced by shuffles.
template <int D>
__device__ void lds_tri_inverse(const double (*sL)[D + 1], double (*sI)[D + 1], int l) {
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  for (int i = ty; i < l; i += 16)
    for (int k = tx; k < l; k += 16) sI[i][k] = 0.0;
  __syncthreads();
  for (int i = 0; i < l; ++i) {
    const double d = sL[i][i];
    for (int c = ty; c <= i; c += 16) {
      double v = 0.0;
      for (int k = c + tx; k < i; k += 16) v += sL[i][k] * sI[k][c];
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 1);
      if (tx == 0) sI[i][c] = (d > 0.0) ? (((c == i) ? 1.0 : 0.0) - v) / d : 0.0;
    }
    __syncthreads();
  }
}

// Cyclic Jacobi on the symmetric sG (n x n): sG ends diagonal (the
// eigenvalues), sV holds the eigenvectors as columns. Round-robin pairing
// over n rounded up to even (the extra slot idles): in each round every index
// is in at most one pair, so the rotations of a round commute and
// G <- J^T G J is applied as a column pass then a row pass. Sweeps stop when
// the squared off-diagonal mass is below 1e-26 of the total (1e-13 in norm)
// or after 30 sweeps.
template <int D>
__device__ void lds_jacobi(double (*sG)[D + 1], double (*sV)[D + 1], int n) {
  __shared__ double sC[D / 2 + 1], sS[D / 2 + 1];
  __shared__ int sP[D / 2 + 1], sQ[D / 2 + 1];
  __shared__ double sOff, sTot, sRedO[4], sRedT[4];
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int ne = n + (n & 1), np = ne / 2;
  for (int i = ty; i < n; i += 16)
    for (int j = tx; j < n; j += 16) sV[i][j] = (i == j) ? 1.0 : 0.0;
  __syncthreads();
  for (int sweep = 0; sweep < 30; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (int i = ty; i < n; i += 16)
      for (int j = tx; j < n; j += 16) {
        const double v = sG[i][j] * sG[i][j];
        tot += v;
        if (i != j) off += v;
      }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      tot += __shfl_xor(tot, o);
    }
    if ((t & 63) == 0) { sRedO[t >> 6] = off; sRedT[t >> 6] = tot; }
    __syncthreads();
    if (t == 0) {
      sOff = ((sRedO[0] + sRedO[1]) + sRedO[2]) + sRedO[3];
      sTot = ((sRedT[0] + sRedT[1]) + sRedT[2]) + sRedT[3];
    }
    __syncthreads();
    if (!(sOff > 1e-26 * sTot)) break;
    for (int round = 0; round < ne - 1; ++round) {
      for (int pi = t; pi < np; pi += 256) {
        auto slot = [&](int x) { return x == 0 ? 0 : 1 + (x - 1 + round) % (ne - 1); };
        int p = slot(pi), q = slot(ne - 1 - pi);
        if (p > q) { const int tmp = p; p = q; q = tmp; }
        double c = 1.0, sn = 0.0;
        if (q < n) {
          const double apq = sG[p][q], app = sG[p][p], aqq = sG[q][q];
          if (apq != 0.0) {
            const double theta = (aqq - app) / (2.0 * apq);
            const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(tt * tt + 1.0);
            sn = tt * c;
          }
        } else {
          q = -1;   // the idle slot
        }
        sP[pi] = p; sQ[pi] = q; sC[pi] = c; sS[pi] = sn;
      }
      __syncthreads();
      // (loops over compile-time bounds with guards, so the LDS reads of a
      // thread are issued together)
#pragma unroll
      for (int k = 0; k < (D / 2 + 15) / 16; ++k) {   // columns: G <- G J, V <- V J
        const int pi = ty + 16 * k;
        if (pi >= np) break;
        const int p = sP[pi], q = sQ[pi];
        if (q < 0) continue;
        const double c = sC[pi], sn = sS[pi];
#pragma unroll
        for (int m = 0; m < (D + 15) / 16; ++m) {
          const int i = tx + 16 * m;
          if (i >= n) break;
          const double gp = sG[i][p], gq = sG[i][q];
          const double vp = sV[i][p], vq = sV[i][q];
          sG[i][p] = c * gp - sn * gq;
          sG[i][q] = sn * gp + c * gq;
          sV[i][p] = c * vp - sn * vq;
          sV[i][q] = sn * vp + c * vq;
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < (D / 2 + 15) / 16; ++k) {   // rows: G <- J^T G
        const int pi = ty + 16 * k;
        if (pi >= np) break;
        const int p = sP[pi], q = sQ[pi];
        if (q < 0) continue;
        const double c = sC[pi], sn = sS[pi];
#pragma unroll
        for (int m = 0; m < (D + 15) / 16; ++m) {
          const int j = tx + 16 * m;
          if (j >= n) break;
          const double gp = sG[p][j], gq = sG[q][j];
          sG[p][j] = c * gp - sn * gq;
          sG[q][j] = sn * gp + c * gq;
        }
      }
      __syncthreads();
    }
  }
}

// sOrder[k] = index of the k-th largest diagonal entry of sG (ties by index)
template <int D>
__device__ void lds_eig_order(const double (*sG)[D + 1], int n, int* sOrder) {
  for (int i = threadIdx.x; i < n; i += 256) {
    const double lt = sG[i][i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const double lj = sG[j][j];
      rank += (lj > lt || (lj == lt && j < i)) ? 1 : 0;
    }
    sOrder[rank] = i;
  }
  __syncthreads();
}

// ---- T = L^{-T} for G = L L^T (one workgroup) -------------------------------
// Gaussian elimination without pivoting on [G | I] (G is symmetric positive
// semi-definite): after step j every row i > j has had f = G[i][j] / G[j][j]
// times row j subtracted, so E G = U with E = L1^{-1} for G = L1 D L1^T
// (L1 unit lower triangular). The Cholesky factor is L = L1 D^{1/2}, hence
// L^{-1} = D^{-1/2} E and T[k][j] = E[j][k] / sqrt(D[j]) for k <= j. A
// dependent column (pivot at or below 1e-28 of the largest diagonal entry)
// eliminates nothing and gets a zero column of T, so Q = Y T has a zero
// column there. One barrier per pivot.
__global__ __launch_bounds__(256) void k_chol_inv(const double* __restrict__ G, int l, double* __restrict__ T) {
  __shared__ double sA[LR_MAXL][LR_MAXL + 1];
  __shared__ double sE[LR_MAXL][LR_MAXL + 1];
  __shared__ double sR[LR_MAXL];   // D[j]^{-1/2}, 0 for a dependent column
  __shared__ double sRed[4];
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  double m = 0.0;
  for (int i = ty; i < l; i += 16)
    for (int k = tx; k < l; k += 16) {
      const double v = G[i * l + k];
      sA[i][k] = v;
      sE[i][k] = (i == k) ? 1.0 : 0.0;
      if (i == k) m = fmax(m, v);
    }
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  if ((t & 63) == 0) sRed[t >> 6] = m;
  __syncthreads();
  const double tol = 1e-28 * fmax(fmax(sRed[0], sRed[1]), fmax(sRed[2], sRed[3]));
  for (int j = 0; j < l; ++j) {
    const double d = sA[j][j];
    const bool ok = d > tol && d > 0.0;
    const double inv = ok ? 1.0 / d : 0.0;
    for (int i = j + 1 + ty; i < l; i += 16) {
      const double f = sA[i][j] * inv;
      for (int k = j + 1 + tx; k < l; k += 16) sA[i][k] -= f * sA[j][k];
      for (int k = tx; k <= j; k += 16) sE[i][k] -= f * sE[j][k];
    }
    if (t == 0) sR[j] = ok ? 1.0 / sqrt(d) : 0.0;
    __syncthreads();
  }
  for (int k = ty; k < l; k += 16)
    for (int j = tx; j < l; j += 16) T[k * l + j] = (k <= j) ? sE[j][k] * sR[j] : 0.0;
}

// ---- eigen-decomposition of the Rayleigh-Ritz Gram (one workgroup) ----------
// The top r eigenpairs (descending) give M1[:, i] = u_i sqrt(sigma_i),
// M2[:, i] = u_i / sqrt(sigma_i) (0 if sigma_i = 0), sigma_i = sqrt(max(lambda_i, 0)).
__global__ __launch_bounds__(256) void k_jacobi_eig(const double* __restrict__ Gin, int l, int r,
                                                     double* __restrict__ M1, double* __restrict__ M2,
                                                     float* __restrict__ sigma) {
  __shared__ double sG[LR_MAXL][LR_MAXL + 1];
  __shared__ double sV[LR_MAXL][LR_MAXL + 1];
  __shared__ int sOrder[LR_MAXL];
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  for (int i = ty; i < l; i += 16)
    for (int j = tx; j < l; j += 16) sG[i][j] = Gin[i * l + j];
  __syncthreads();
  lds_jacobi<LR_MAXL>(sG, sV, l);
  lds_eig_order<LR_MAXL>(sG, l, sOrder);
  for (int i = ty; i < l; i += 16)
    for (int k = tx; k < r; k += 16) {
      const int col = sOrder[k];
      const double sg = sqrt(fmax(sG[col][col], 0.0));
      const double h = sqrt(sg);
      M1[i * r + k] = sV[i][col] * h;
      M2[i * r + k] = (h > 0.0) ? sV[i][col] / h : 0.0;
      if (i == 0) sigma[k] = (float)sg;
    }
}

// ---- out = X S (X [M, l] float32, S [l, c] float64), or its transpose --------
// Workgroup: 16 rows of X staged in LDS; thread -> (row, column) pairs. The
// rows are read into LDS before any output is written, so out may alias X
// when c == l and the output is not transposed.
__global__ __launch_bounds__(256) void k_right_mul(const float* X, int64_t M, int l,
                                                   const double* __restrict__ S, int c,
                                                   float* out, int transposed) {
  __shared__ double sS[LR_MAXL * LR_MAXL];
  __shared__ float sX[16][LR_MAXL + 1];
  const int t = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  for (int e = t; e < l * c; e += 256) sS[e] = S[e];
  for (int e = t; e < 16 * l; e += 256) {
    const int rr = e / l, i = e % l;
    const int64_t m = m0 + rr;
    sX[rr][i] = (m < M) ? X[m * l + i] : 0.0f;
  }
  __syncthreads();
  for (int e = t; e < 16 * c; e += 256) {
    const int rr = e / c, j = e % c;
    const int64_t m = m0 + rr;
    if (m >= M) continue;
    double v = 0.0;
    for (int i = 0; i < l; ++i) v += (double)sX[rr][i] * sS[i * c + j];
    if (transposed) out[(int64_t)j * M + m] = (float)v;
    else out[m * c + j] = (float)v;
  }
}

// ---- ||R - B A||_F^2: float64 partials per workgroup, fixed-order finish -----
__global__ __launch_bounds__(256) void k_lowrank_sqerr(const float* __restrict__ R, int64_t N, int64_t K,
                                                       const float* __restrict__ B, const float* __restrict__ A,
                                                       int r, double* __restrict__ part) {
  __shared__ double sW[4];
  const int64_t quads = N * K / 4;
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (int64_t)gridDim.x * 256) {
    const int64_t e = 4 * i;
    const int64_t n = e / K, k = e - n * K;
    double d[4] = {0.0, 0.0, 0.0, 0.0};
    for (int j = 0; j < r; ++j) {
      const double b = (double)B[n * r + j];
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(A + (int64_t)j * K + k);
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] += b * (double)a[q];
    }
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(R + e);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double v = (double)x[q] - d[q];
      acc += v * v;
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sW[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = ((sW[0] + sW[1]) + sW[2]) + sW[3];
}

// Fixed-order sum of n partials: lane l adds partials l, l + 64, ... in
// order, then the 64 lane sums are added pairwise (a fixed tree). One thread
// adding all 1024 in sequence took 59 us.
__global__ __launch_bounds__(64) void k_sum_doubles(const double* __restrict__ part, int n, double* __restrict__ out) {
  double v = 0.0;
  for (int i = threadIdx.x; i < n; i += 64) v += part[i];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = v + __shfl_xor(v, m);
  if (threadIdx.x == 0) *out = v;
}

static unsigned grid_for(int64_t items, int64_t per_wg, int64_t cap) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cap, (items + per_wg - 1) / per_wg));
}

constexpr int SKINNY_SPLITS = 16;   // most contraction slices of a tall-skinny product
constexpr int GRAM_PARTS = 64;
constexpr int SQERR_WGS = 1024;

}  // namespace

int lowrank_max_l() { return LR_MAXL; }

hipError_t launch_lowrank_sub(const float* W, int64_t N, int64_t K, const float* B, const float* A, int r,
                              float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_lowrank_sub, dim3(grid_for(N * K / 4, 256, 8192)), dim3(256), 0, s, W, N, K, B, A, r, out);
  return hipGetLastError();
}

hipError_t launch_residual(const float* W, const uint16_t* Wd, int64_t n, float* R, hipStream_t s) {
  hipLaunchKernelGGL(k_residual, dim3(grid_for(n / 4, 256, 8192)), dim3(256), 0, s, W, Wd, n, R);
  return hipGetLastError();
}

// Workspace of the rank-r SVD, in floats: Y [N, l], Z [K, l], split partials
// [S, max(N, K), l]; then float64: Gram partials, G, L, M1, M2.
size_t svd_ws_bytes(int64_t N, int64_t K, int l, int r) {
  const int64_t mx = std::max(N, K);
  size_t f = (size_t)(N * l + K * l + (int64_t)SKINNY_SPLITS * mx * l);
  f = (f + 1) & ~(size_t)1;   // float64 alignment
  const size_t d = (size_t)GRAM_PARTS * l * l + 2 * (size_t)l * l + 2 * (size_t)l * r + SQERR_WGS;
  return f * sizeof(float) + d * sizeof(double);
}

namespace {
struct SvdWs {
  float *Y, *Z, *part;
  double *gpart, *G, *L, *M1, *M2, *sq;
};
SvdWs carve(void* ws, int64_t N, int64_t K, int l, int r) {
  SvdWs w;
  float* f = (float*)ws;
  const int64_t mx = std::max(N, K);
  w.Y = f; f += N * l;
  w.Z = f; f += K * l;
  w.part = f; f += (int64_t)SKINNY_SPLITS * mx * l;
  size_t used = (size_t)(f - (float*)ws);
  used = (used + 1) & ~(size_t)1;
  double* d = (double*)((float*)ws + used);
  w.gpart = d; d += (size_t)GRAM_PARTS * l * l;
  w.G = d; d += (size_t)l * l;
  w.L = d; d += (size_t)l * l;
  w.M1 = d; d += (size_t)l * r;
  w.M2 = d; d += (size_t)l * r;
  w.sq = d;
  return w;
}

#define LR_CHECK() do { hipError_t e_ = hipGetLastError(); if (e_ != hipSuccess) return e_; } while (0)

// Y [M, l] <- orthonormal basis of its columns (CholQR twice)
hipError_t orthonormalise(float* Y, int64_t M, int l, const SvdWs& w, hipStream_t s) {
  const int parts = (int)std::min<int64_t>(GRAM_PARTS, (M + 31) / 32);
  const int64_t rows = (M + parts - 1) / parts;
  for (int pass = 0; pass < 2; ++pass) {
    hipLaunchKernelGGL(k_gram_partial, dim3(parts), dim3(256), 0, s, Y, M, l, rows, w.gpart);
    hipLaunchKernelGGL(k_gram_finish, dim3(grid_for(l * l, 256, 64)), dim3(256), 0, s, w.gpart, parts, l * l, w.G);
    hipLaunchKernelGGL(k_chol_inv, dim3(1), dim3(256), 0, s, w.G, l, w.L);
    hipLaunchKernelGGL(k_right_mul, dim3((unsigned)((M + 15) / 16)), dim3(256), 0, s, Y, M, l, w.L, l, Y, 0);
    LR_CHECK();
  }
  return hipSuccess;
}

template <bool TRANS, int TN>
void launch_skinny_tn(const float* X, int64_t M, int64_t C, const float* V, int l, int64_t kslice, int slices,
                      float* part, hipStream_t s) {
  const int64_t rows_out = TRANS ? C : M;
  const dim3 grid((unsigned)((rows_out + 127) / 128), (unsigned)slices);
  hipLaunchKernelGGL((k_skinny_gemm<TRANS, TN>), grid, dim3(256), 0, s, X, M, C, V, l, kslice, part);
}

// out = X V (trans = false, [M, l]) or X^T V (trans = true, [C, l]) for X [M, C]:
// enough contraction slices for about 512 workgroups, summed in a fixed order.
hipError_t skinny(const float* X, int64_t M, int64_t C, const float* V, int l, bool trans, float* out,
                  const SvdWs& w, hipStream_t s) {
  const int64_t rows_out = trans ? C : M, kc = trans ? M : C;
  const int64_t tiles = (rows_out + 127) / 128;
  int slices = (int)std::min<int64_t>(SKINNY_SPLITS, std::max<int64_t>(1, (512 + tiles - 1) / tiles));
  int64_t kslice = (kc + slices - 1) / slices;
  kslice = (kslice + 31) / 32 * 32;
  slices = (int)((kc + kslice - 1) / kslice);
  const int tn = ((l + 31) / 32) * 4;
  if (trans) {
    if (tn == 4) launch_skinny_tn<true, 4>(X, M, C, V, l, kslice, slices, w.part, s);
    else if (tn == 8) launch_skinny_tn<true, 8>(X, M, C, V, l, kslice, slices, w.part, s);
    else launch_skinny_tn<true, 12>(X, M, C, V, l, kslice, slices, w.part, s);
  } else {
    if (tn == 4) launch_skinny_tn<false, 4>(X, M, C, V, l, kslice, slices, w.part, s);
    else if (tn == 8) launch_skinny_tn<false, 8>(X, M, C, V, l, kslice, slices, w.part, s);
    else launch_skinny_tn<false, 12>(X, M, C, V, l, kslice, slices, w.part, s);
  }
  hipLaunchKernelGGL(k_sum_splits, dim3(grid_for(rows_out * l, 256, 4096)), dim3(256), 0, s, w.part, slices,
                     rows_out * l, out);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_svd_lowrank(const float* R, int64_t N, int64_t K, int r, int l, int power_iters,
                              const float* omega, float* B, float* A, float* sigma, void* ws, hipStream_t s) {
  const SvdWs w = carve(ws, N, K, l, r);
  hipError_t e;
  if ((e = skinny(R, N, K, omega, l, false, w.Y, w, s)) != hipSuccess) return e;
  if ((e = orthonormalise(w.Y, N, l, w, s)) != hipSuccess) return e;
  for (int it = 0; it < power_iters; ++it) {
    // Y <- orth(R R^T Y): the float64 Gram of CholQR (applied twice) takes the
    // squared condition number of R R^T Y
    if ((e = skinny(R, N, K, w.Y, l, true, w.Z, w, s)) != hipSuccess) return e;
    if ((e = skinny(R, N, K, w.Z, l, false, w.Y, w, s)) != hipSuccess) return e;
    if ((e = orthonormalise(w.Y, N, l, w, s)) != hipSuccess) return e;
  }
  // Rayleigh-Ritz: Z = R^T Y, eigen-decomposition of Z^T Z
  if ((e = skinny(R, N, K, w.Y, l, true, w.Z, w, s)) != hipSuccess) return e;
  const int parts = (int)std::min<int64_t>(GRAM_PARTS, (K + 31) / 32);
  hipLaunchKernelGGL(k_gram_partial, dim3(parts), dim3(256), 0, s, w.Z, K, l, (K + parts - 1) / parts, w.gpart);
  hipLaunchKernelGGL(k_gram_finish, dim3(grid_for(l * l, 256, 64)), dim3(256), 0, s, w.gpart, parts, l * l, w.G);
  hipLaunchKernelGGL(k_jacobi_eig, dim3(1), dim3(256), 0, s, w.G, l, r, w.M1, w.M2, sigma);
  hipLaunchKernelGGL(k_right_mul, dim3((unsigned)((N + 15) / 16)), dim3(256), 0, s, w.Y, N, l, w.M1, r, B, 0);
  hipLaunchKernelGGL(k_right_mul, dim3((unsigned)((K + 15) / 16)), dim3(256), 0, s, w.Z, K, l, w.M2, r, A, 1);
  return hipGetLastError();
}

hipError_t launch_lowrank_sqerr(const float* R, int64_t N, int64_t K, const float* B, const float* A, int r,
                                double* out, void* ws, hipStream_t s) {
  double* part = (double*)ws;
  const unsigned g = grid_for(N * K / 4, 256, SQERR_WGS);
  hipLaunchKernelGGL(k_lowrank_sqerr, dim3(g), dim3(256), 0, s, R, N, K, B, A, r, part);
  hipLaunchKernelGGL(k_sum_doubles, dim3(1), dim3(64), 0, s, part, (int)g, out);
  return hipGetLastError();
}

size_t sqerr_ws_bytes() { return SQERR_WGS * sizeof(double); }

namespace {
__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
}  // namespace

size_t loftq_ws_bytes(int64_t N, int64_t K, int r, int l, bool dq) {
  const int64_t n = N * K;
  size_t b = align256((size_t)n * sizeof(float)) + align256((size_t)n * sizeof(uint16_t));
  if (dq) b += align256(double_quant_ws_doubles(n / 64) * sizeof(double));
  b += align256(svd_ws_bytes(N, K, l, r)) + align256(sqerr_ws_bytes());
  return b;
}

hipError_t launch_loftq(const float* W, int64_t N, int64_t K, bool dq, int r, int l, int steps, int power_iters,
                        const float* omega, uint8_t* codes, float* absmax, uint8_t* absmax_q, float* dq_scale,
                        float* dq_mean, float* B, float* A, float* sigma, double* objectives, void* ws,
                        hipStream_t s) {
  const int64_t n = N * K, n_blocks = n / 64;
  char* p = (char*)ws;
  float* Wt = (float*)p;               // W - B A, then the residual R
  p += align256((size_t)n * sizeof(float));
  uint16_t* Wd = (uint16_t*)p;         // the layer's bf16 weight
  p += align256((size_t)n * sizeof(uint16_t));
  double* dq_ws = (double*)p;
  if (dq) p += align256(double_quant_ws_doubles(n_blocks) * sizeof(double));
  void* svd_ws = p;
  p += align256(svd_ws_bytes(N, K, l, r));
  void* sq_ws = p;

  hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(N * r, 256, 1024)), dim3(256), 0, s, B, N * (int64_t)r);
  hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(K * r, 256, 1024)), dim3(256), 0, s, A, K * (int64_t)r);
  LR_CHECK();
  QWeight q{};
  q.format = LQ_FMT_NF4;
  q.N = N;
  q.K = K;
  q.codes = codes;
  if (dq) q.qc = QConst{nullptr, absmax_q, dq_scale, dq_mean};
  else q.qc = QConst{absmax, nullptr, nullptr, nullptr};
  hipError_t e;
  for (int t = 0; t < steps; ++t) {
    const float* src = W;              // the adapter starts at zero
    if (t > 0) {
      if ((e = launch_lowrank_sub(W, N, K, B, A, r, Wt, s)) != hipSuccess) return e;
      src = Wt;
    }
    if ((e = launch_quantize_nf4(src, LQ_F32, n_blocks, codes, absmax, s)) != hipSuccess) return e;
    if (dq && (e = launch_double_quant(absmax, n_blocks, absmax_q, dq_scale, dq_mean, dq_ws, s)) != hipSuccess)
      return e;
    if ((e = launch_dequant(q, Wd, s)) != hipSuccess) return e;
    if ((e = launch_residual(W, Wd, n, Wt, s)) != hipSuccess) return e;
    if ((e = launch_svd_lowrank(Wt, N, K, r, l, power_iters, omega, B, A, sigma, svd_ws, s)) != hipSuccess) return e;
    if (objectives && (e = launch_lowrank_sqerr(Wt, N, K, B, A, r, objectives + t, sq_ws, s)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// ===========================================================================
// LoRAQuant-style quantization of an adapter (LoRAQuant page, method overview
// and key design): SVD reparameterization B A = B' A' with B' = U S^(1/2),
// A' = S^(1/2) V^T, the important components (by singular value) at a higher
// width, the rest at an ultra-low width, each component vector quantized in
// the codebook format with its own weighted Lloyd-Max codebook of its width.
//
// The SVD needs only r x r work: with G_B = B^T B, G_A = A A^T = L_A L_A^T
// and S = L_A^T G_B L_A = W diag(sigma^2) W^T,
//   B' = B (L_A W sigma^(-1/2)),  A' = (sigma^(1/2) W^T L_A^(-1)) A,
// so that B' A' = B A, B'^T B' = A' A'^T = diag(sigma).
// ===========================================================================
namespace {

constexpr int LQ_D = LQ_LORAQUANT_MAX_R;

__global__ __launch_bounds__(256) void k_adapter_core(const double* __restrict__ GB, const double* __restrict__ GA,
                                                      int r, double rho, int h_fixed, int bits_hi, int bits_lo,
                                                      double* __restrict__ MBt, double* __restrict__ MA,
                                                      float* __restrict__ sigma, int32_t* __restrict__ h_out,
                                                      uint8_t* __restrict__ row_bits) {
  __shared__ double sA[LQ_D][LQ_D + 1];   // G_A (destroyed), then G_B L_A, then W
  __shared__ double sL[LQ_D][LQ_D + 1];   // L_A
  __shared__ double sI[LQ_D][LQ_D + 1];   // L_A^{-1}
  __shared__ double sS[LQ_D][LQ_D + 1];   // G_B, then S (diagonalised)
  __shared__ int sOrder[LQ_D];
  __shared__ double sSig[LQ_D];
  __shared__ double sRed[4];
  __shared__ int sH;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  double m = 0.0;
  for (int i = ty; i < r; i += 16)
    for (int k = tx; k < r; k += 16) {
      const double a = GA[i * r + k];
      sA[i][k] = a;
      sS[i][k] = GB[i * r + k];
      if (i == k) m = fmax(m, a);
    }
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  if ((t & 63) == 0) sRed[t >> 6] = m;
  __syncthreads();
  const double tol = 1e-28 * fmax(fmax(sRed[0], sRed[1]), fmax(sRed[2], sRed[3]));
  lds_cholesky<LQ_D>(sA, sL, r, tol);
  lds_tri_inverse<LQ_D>(sL, sI, r);
  for (int i = ty; i < r; i += 16)          // sA = G_B L_A
    for (int j = tx; j < r; j += 16) {
      double v = 0.0;
      for (int k = j; k < r; ++k) v += sS[i][k] * sL[k][j];
      sA[i][j] = v;
    }
  __syncthreads();
  for (int i = ty; i < r; i += 16)          // sS = L_A^T (G_B L_A)
    for (int j = tx; j < r; j += 16) {
      double v = 0.0;
      for (int k = i; k < r; ++k) v += sL[k][i] * sA[k][j];
      sS[i][j] = v;
    }
  __syncthreads();
  for (int i = ty; i < r; i += 16)          // symmetrise
    for (int j = tx; j < i; j += 16) {
      const double v = 0.5 * (sS[i][j] + sS[j][i]);
      sS[i][j] = v;
      sS[j][i] = v;
    }
  __syncthreads();
  lds_jacobi<LQ_D>(sS, sA, r);              // sA = W
  lds_eig_order<LQ_D>(sS, r, sOrder);
  for (int k = t; k < r; k += 256) {
    const double sg = sqrt(fmax(sS[sOrder[k]][sOrder[k]], 0.0));
    sSig[k] = sg;
    sigma[k] = (float)sg;
  }
  __syncthreads();
  if (t == 0) {
    int h;
    if (h_fixed >= 0) {
      h = min(h_fixed, r);
    } else {
      // energies of the float32 singular values, summed in order
      double tot = 0.0;
      for (int k = 0; k < r; ++k) { const double f = (double)(float)sSig[k]; tot += f * f; }
      if (tot == 0.0) {
        h = 0;
      } else {
        double c = 0.0;
        h = r;
        for (int k = 0; k < r; ++k) {
          const double f = (double)(float)sSig[k];
          c += f * f;
          if (c >= rho * tot) { h = k + 1; break; }
        }
      }
    }
    sH = h;
    *h_out = h;
  }
  __syncthreads();
  const int h = sH;
  for (int k = ty; k < r; k += 16)
    for (int j = tx; j < r; j += 16) {
      const int col = sOrder[k];
      const double sg = sSig[k];
      const double rs = sqrt(sg);
      double b = 0.0;
      for (int q = 0; q <= j; ++q) b += sL[j][q] * sA[q][col];       // (L_A W)[j][col]
      double a = 0.0;
      for (int q = j; q < r; ++q) a += sA[q][col] * sI[q][j];        // (W^T L_A^{-1})[col][j]
      MBt[k * r + j] = (rs > 0.0) ? b / rs : 0.0;                    // M_B^T[k][j]
      MA[k * r + j] = rs * a;                                         // M_A[k][j]
    }
  for (int k = t; k < r; k += 256) row_bits[k] = (uint8_t)((k < h) ? bits_hi : bits_lo);
}

// out[i][c] = sum_j M[i][j] X(j, c) for i < r, c < C, summed in float64;
// X(j, c) = X[j C + c] (X [r, C]) or X[c r + j] (transposed: X [C, r]).
__global__ __launch_bounds__(256) void k_small_left(const double* __restrict__ M, int r,
                                                    const float* __restrict__ X, int64_t C, int trans,
                                                    float* __restrict__ out) {
  __shared__ double sM[LQ_D * LQ_D];
  __shared__ float sX[LQ_D][257];
  const int t = threadIdx.x;
  const int64_t c = (int64_t)blockIdx.x * 256 + t;
  for (int e = t; e < r * r; e += 256) sM[e] = M[e];
  for (int j = 0; j < r; ++j) sX[j][t] = (c < C) ? (trans ? X[c * r + j] : X[(int64_t)j * C + c]) : 0.0f;
  __syncthreads();
  if (c >= C) return;
  for (int i = 0; i < r; ++i) {
    double v = 0.0;
    for (int j = 0; j < r; ++j) v += sM[i * r + j] * (double)sX[j][t];
    out[(int64_t)i * C + c] = (float)v;
  }
}

// Component i: the entry of largest magnitude in row i of A' (the first on
// ties) is made positive; row i of B'^T flips with it.
__global__ __launch_bounds__(256) void k_sign_fix(float* __restrict__ Ap, int64_t K, float* __restrict__ Bpt,
                                                  int64_t N) {
  __shared__ float sV[4];
  __shared__ int64_t sK[4];
  __shared__ int sFlip;
  const int t = threadIdx.x;
  const int64_t i = blockIdx.x;
  float best = -1.0f;
  int64_t bk = 0;
  for (int64_t k = t; k < K; k += 256) {
    const float v = fabsf(Ap[i * K + k]);
    if (v > best) { best = v; bk = k; }   // k increases per thread: the first maximum stays
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o);
    const int64_t ok = __shfl_xor(bk, o);
    if (ov > best || (ov == best && ok < bk)) { best = ov; bk = ok; }
  }
  if ((t & 63) == 0) { sV[t >> 6] = best; sK[t >> 6] = bk; }
  __syncthreads();
  if (t == 0) {
    float b = sV[0];
    int64_t kk = sK[0];
    for (int w = 1; w < 4; ++w)
      if (sV[w] > b || (sV[w] == b && sK[w] < kk)) { b = sV[w]; kk = sK[w]; }
    sFlip = Ap[i * K + kk] < 0.0f;
  }
  __syncthreads();
  if (!sFlip) return;
  for (int64_t k = t; k < K; k += 256) Ap[i * K + k] = -Ap[i * K + k];
  for (int64_t n = t; n < N; n += 256) Bpt[i * N + n] = -Bpt[i * N + n];
}

__global__ void k_row_offsets(const uint8_t* __restrict__ row_bits, int r, int64_t K, int64_t N,
                              int64_t* __restrict__ offA, int64_t* __restrict__ offB) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int64_t a = 0, b = 0;
  for (int i = 0; i < r; ++i) {
    offA[i] = a;
    offB[i] = b;
    a += K * row_bits[i] / 8;
    b += N * row_bits[i] / 8;
  }
  offA[r] = a;
  offB[r] = b;
}

__global__ __launch_bounds__(256) void k_transpose_f32(const float* __restrict__ in, int rows, int64_t cols,
                                                       float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over in [rows, cols]
  if (e >= (int64_t)rows * cols) return;
  const int64_t i = e / cols, c = e % cols;
  out[c * rows + i] = in[e];
}

struct LqWs {
  float *At, *Ap, *Bpt;
  double *gpart, *GB, *GA, *MBt, *MA;
};
LqWs carve_lq(void* ws, int64_t N, int64_t K, int r) {
  LqWs w;
  char* p = (char*)ws;
  w.At = (float*)p; p += align256((size_t)K * r * sizeof(float));
  w.Ap = (float*)p; p += align256((size_t)K * r * sizeof(float));
  w.Bpt = (float*)p; p += align256((size_t)N * r * sizeof(float));
  w.gpart = (double*)p; p += align256((size_t)GRAM_PARTS * r * r * sizeof(double));
  w.GB = (double*)p; p += align256((size_t)r * r * sizeof(double));
  w.GA = (double*)p; p += align256((size_t)r * r * sizeof(double));
  w.MBt = (double*)p; p += align256((size_t)r * r * sizeof(double));
  w.MA = (double*)p;
  return w;
}

hipError_t gram(const float* Y, int64_t M, int l, double* part, double* G, hipStream_t s) {
  const int parts = (int)std::min<int64_t>(GRAM_PARTS, (M + 31) / 32);
  hipLaunchKernelGGL(k_gram_partial, dim3(parts), dim3(256), 0, s, Y, M, l, (M + parts - 1) / parts, part);
  hipLaunchKernelGGL(k_gram_finish, dim3(grid_for(l * l, 256, 64)), dim3(256), 0, s, part, parts, l * l, G);
  return hipGetLastError();
}

}  // namespace

size_t loraquant_ws_bytes(int64_t N, int64_t K, int r) {
  return 2 * align256((size_t)K * r * sizeof(float)) + align256((size_t)N * r * sizeof(float)) +
         align256((size_t)GRAM_PARTS * r * r * sizeof(double)) + 4 * align256((size_t)r * r * sizeof(double));
}

hipError_t launch_loraquant(const float* B, const float* A, int64_t N, int64_t K, int r, double rho, int h_fixed,
                            int bits_hi, int bits_lo, uint8_t* codes_a, float* absmax_a, uint8_t* codes_b,
                            float* absmax_b, uint8_t* row_bits, int64_t* offsets_a, int64_t* offsets_b,
                            float* levels_a, float* thresholds_a, float* levels_b, float* thresholds_b,
                            float* sigma, int32_t* h_out, float* Ap_out, float* Bpt_out, void* ws, hipStream_t s) {
  LqWs w = carve_lq(ws, N, K, r);
  float* Ap = Ap_out ? Ap_out : w.Ap;
  float* Bpt = Bpt_out ? Bpt_out : w.Bpt;
  hipError_t e;
  if ((e = gram(B, N, r, w.gpart, w.GB, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_transpose_f32, dim3((unsigned)((K * r + 255) / 256)), dim3(256), 0, s, A, r, K, w.At);
  if ((e = gram(w.At, K, r, w.gpart, w.GA, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_adapter_core, dim3(1), dim3(256), 0, s, w.GB, w.GA, r, rho, h_fixed, bits_hi, bits_lo,
                     w.MBt, w.MA, sigma, h_out, row_bits);
  hipLaunchKernelGGL(k_small_left, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, w.MA, r, A, K, 0, Ap);
  hipLaunchKernelGGL(k_small_left, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, w.MBt, r, B, N, 1, Bpt);
  hipLaunchKernelGGL(k_sign_fix, dim3((unsigned)r), dim3(256), 0, s, Ap, K, Bpt, N);
  hipLaunchKernelGGL(k_row_offsets, dim3(1), dim3(64), 0, s, row_bits, r, K, N, offsets_a, offsets_b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // per-component codebooks (weighted Lloyd-Max, 100 iterations at most), then quantization
  if ((e = launch_lloyd(Ap, LQ_F32, r, K, row_bits, 100, levels_a, thresholds_a, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_lloyd(Bpt, LQ_F32, r, N, row_bits, 100, levels_b, thresholds_b, nullptr, s)) != hipSuccess) return e;
  if ((e = launch_quantize_codebook(Ap, LQ_F32, r, K, row_bits, offsets_a, thresholds_a, codes_a, absmax_a, s)) !=
      hipSuccess)
    return e;
  return launch_quantize_codebook(Bpt, LQ_F32, r, N, row_bits, offsets_b, thresholds_b, codes_b, absmax_b, s);
}

}  // namespace lq
