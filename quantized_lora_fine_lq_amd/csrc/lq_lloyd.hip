// Weighted Lloyd-Max learner for per-output-channel codebooks (LowRA,
// section 5, "mapping and threshold learner"): each output channel's levels
// and thresholds minimise that channel's weighted mean squared error, every
// element weighted by the absmax of its 64-block; thresholds start from the
// NormalFloat thresholds of the channel's width; each iteration takes the
// weighted centroid of every interval as its level, then the midpoints of
// adjacent levels as the new thresholds; the learner stops at the iteration
// limit or when the error stops decreasing, and keeps the last computed
// levels and thresholds.
//
// One workgroup per row. The row's normalised values x = w / c (float32, as
// the quantizer computes them) are sorted once in LDS (bitonic network on
// 64-bit keys: order-preserving bits of x above the element index, so the
// order is total and each element finds its block constant again). With the
// values sorted, an interval of thresholds is a contiguous range of
// positions, so an iteration needs no pass over the row:
//   * the position of threshold T (the number of values <= T) is found by a
//     16-ary search over the last value of each 16-element segment, then a
//     vote inside the segment;
//   * the sums of w, w*x and w*x^2 over an interval are added directly in
//     float64 from per-segment sums and the partial segments at both ends, in
//     a fixed order (no differences of prefix sums, so a bin's sum carries
//     only its own rounding).
// The comparison x <= T with T in float64 is made in float32 against the
// largest float32 not above T, which decides every float32 x the same way.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lq_device.h"
#include "lq_internal.h"

namespace lq {
namespace {

constexpr uint32_t kPadHi = 0xFFFFFFFFu;   // high key word of padding slots

// order-preserving map of a float32 to uint32 (-0 sorts just below +0)
__device__ __forceinline__ uint32_t f32_order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t s = (uint32_t)(key >> 32);
  if (s == kPadHi) return INFINITY;
  return __uint_as_float((s & 0x80000000u) ? (s & 0x7FFFFFFFu) : ~s);
}

// LDS slot of sorted position p: the low 4 bits are XORed with bits 4..7, so
// that 64 lanes reading 16 consecutive keys each (lane stride 128 bytes) hit
// distinct banks; the slot stays inside p's aligned group of 16.
__device__ __forceinline__ int kslot(int p) { return p ^ ((p >> 4) & 15); }

__device__ __forceinline__ void cmp_swap(uint64_t& a, uint64_t& b, bool ascending) {
  const uint64_t lo = a < b ? a : b;
  const uint64_t hi = a < b ? b : a;
  a = ascending ? lo : hi;
  b = ascending ? hi : lo;
}

// G consecutive substages (strides j, j/2, ..., j >> (G-1), all >= 16) of the
// bitonic stage `size`, on sets of 2^G keys that these substages only ever
// compare among themselves; each thread takes 16 keys (16 >> G sets). Keys
// of sorted position p live in LDS slot kslot(p).
template <int G, int NT>
__device__ __forceinline__ void bitonic_group(uint64_t* s, int lj, int size, int t) {
  constexpr int E = 1 << G;
  constexpr int R = 16 / E;
  const int lb = lj - G + 1;   // lowest position bit that varies within a set
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int q = t + NT * r;
    const int base = ((q >> lb) << (lb + G)) | (q & ((1 << lb) - 1));
    const bool asc = (base & size) == 0;
    uint64_t v[E];
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = s[kslot(base + (m << lb))];
#pragma unroll
    for (int st = G - 1; st >= 0; --st)
#pragma unroll
      for (int m = 0; m < E; ++m)
        if (!(m & (1 << st))) cmp_swap(v[m], v[m | (1 << st)], asc);
#pragma unroll
    for (int m = 0; m < E; ++m) s[kslot(base + (m << lb))] = v[m];
  }
}

// Numbers of sorted values <= Ta and <= Tb, for the 16 lanes of one row group
// (e = lane within the group, gmask = the group's lanes); every lane of the
// group must be active and the results are uniform over the group. A 16-ary
// search over the segment maxima (rounds fixed by NT, the two searches side
// by side), then a vote inside the segment found.
// Invariant per search: segments below lo end <= T; segments from lo + len
// on end > T or do not exist.
template <int NT>
__device__ __forceinline__ void sorted_positions(float Ta, float Tb, const float* sLast,
                                                 const uint64_t* sKey, int e, uint64_t gmask,
                                                 int& pa, int& pb) {
  int la = 0, lb = 0;
#pragma unroll
  for (int len = NT; len > 1;) {
    const int n = len < 16 ? len : 16;
    const int sub = len / n;
    const int ia = la + (e + 1) * sub - 1;
    const int ib = lb + (e + 1) * sub - 1;
    const float va = sLast[ia < NT ? ia : NT - 1];
    const float vb = sLast[ib < NT ? ib : NT - 1];
    const bool qa = (e < n) && (ia < NT) && (va <= Ta);
    const bool qb = (e < n) && (ib < NT) && (vb <= Tb);
    la += __popcll(__ballot(qa) & gmask) * sub;
    lb += __popcll(__ballot(qb) & gmask) * sub;
    len = sub;
  }
  const float xa = key_value(sKey[kslot(min(la, NT - 1) * 16 + e)]);
  const float xb = key_value(sKey[kslot(min(lb, NT - 1) * 16 + e)]);
  pa = la * 16 + ((la < NT) ? __popcll(__ballot(xa <= Ta) & gmask) : 0);
  pb = lb * 16 + ((lb < NT) ? __popcll(__ballot(xb <= Tb) & gmask) : 0);
}

template <typename Tin> __device__ __forceinline__ float load_w(const Tin* p);
template <> __device__ __forceinline__ float load_w<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_w<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_w<_Float16>(const _Float16* p) { return (float)*p; }

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
// Sum over the 16 lanes of a DPP row; every lane of the row ends with the
// same bits (each step adds two operands that its partner adds in the other
// order).
__device__ __forceinline__ double row16_sum(double v) {
  v = v + dpp_f64<DPP_QUAD_XOR1>(v);
  v = v + dpp_f64<DPP_QUAD_XOR2>(v);
  v = v + dpp_f64<DPP_ROW_HALF_MIRROR>(v);
  v = v + dpp_f64<DPP_ROW_MIRROR>(v);
  return v;
}

template <int NT, typename Tin>
__global__ __launch_bounds__(NT) void k_lloyd(const Tin* __restrict__ W, int64_t K,
                                              const uint8_t* __restrict__ row_bits,
                                              int max_iters, LloydInit init,
                                              float* __restrict__ levels,
                                              float* __restrict__ thresholds,
                                              int32_t* __restrict__ iterations) {
  constexpr int KP = NT * 16;   // sorted slots (K padded up)
  __shared__ uint64_t sKey[KP];
  __shared__ double sSeg[3][NT];          // per 16-slot segment: sum w, w x, w x^2
  __shared__ float sLast[NT];             // last (largest) value of each segment
  __shared__ float sAbs[KP / 64];         // block constants of the row
  __shared__ double sBin[2][16][3];       // interval sums, double buffered

  const int t = threadIdx.x, lane = t & 63;
  const int64_t row = blockIdx.x;
  const int nbits = min(max((int)row_bits[row], 1), 4);
  const int nb = 1 << nbits, nT = nb - 1;
  const int Ki = (int)K;

  // ---- load, block absmax, x = w / c, keys --------------------------------
  // thread t takes elements 16t .. 16t+15 (four threads per 64-block) into
  // sorted slots 16t .. 16t+15 (any start order serves the sort)
  uint64_t k[16];
  {
    const int e0 = t * 16;
    // threads past the row read its last 16 elements and zero them, so no
    // load sits behind a branch (the compiler would wait for each one inside it)
    const Tin* Wr = W + row * K + min(e0, Ki - 16);
    float w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = load_w<Tin>(Wr + i);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (e0 >= Ki) w[i] = 0.0f;
      m = fmaxf(m, fabsf(w[i]));
    }
    m = fmaxf(m, dpp_f32<DPP_QUAD_XOR1>(m));
    m = fmaxf(m, dpp_f32<DPP_QUAD_XOR2>(m));
    if (e0 < Ki && (t & 3) == 0) sAbs[t >> 2] = m;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = (m > 0.0f) ? w[i] / m : 0.0f;
      k[i] = (e0 < Ki) ? (((uint64_t)f32_order_bits(x) << 32) | (uint32_t)(e0 + i))
                       : (((uint64_t)kPadHi << 32) | (uint32_t)(e0 + i));
    }
  }

  // ---- bitonic sort, ascending -------------------------------------------
  // stages up to 16 inside each thread's 16 keys (slots 16t .. 16t+15)
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1)
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i ^ j) > i) cmp_swap(k[i], k[i ^ j], (((t * 16 + i) & size) == 0));
  const int sw = t & 15;   // kslot(16t + i) = 16t + (i ^ sw)
  for (int size = 32; size <= KP; size <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sKey[t * 16 + (i ^ sw)] = k[i];
    __syncthreads();
    int lj = 31 - __builtin_clz((unsigned)size) - 1;   // log2 of the first stride
    while (lj >= 4) {
      const int g = min(4, lj - 3);
      if (g == 4) bitonic_group<4, NT>(sKey, lj, size, t);
      else if (g == 3) bitonic_group<3, NT>(sKey, lj, size, t);
      else if (g == 2) bitonic_group<2, NT>(sKey, lj, size, t);
      else bitonic_group<1, NT>(sKey, lj, size, t);
      __syncthreads();
      lj -= g;
    }
    // strides 8 .. 1 inside the thread's own 16 slots
#pragma unroll
    for (int i = 0; i < 16; ++i) k[i] = sKey[t * 16 + (i ^ sw)];
    const bool asc = ((t * 16) & size) == 0;
#pragma unroll
    for (int j = 8; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i ^ j) > i) cmp_swap(k[i], k[i ^ j], asc);
  }

  // ---- segment sums (thread t owns sorted positions 16t .. 16t+15) -------
  {
    double sw0 = 0.0, swx = 0.0, swx2 = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sKey[t * 16 + (i ^ sw)] = k[i];
      if ((uint32_t)(k[i] >> 32) != kPadHi) {
        const double x = (double)key_value(k[i]);
        const double w = (double)sAbs[(uint32_t)k[i] >> 6];
        const double wx = w * x;
        sw0 += w;
        swx += wx;
        swx2 += wx * x;
      }
    }
    sSeg[0][t] = sw0;
    sSeg[1][t] = swx;
    sSeg[2][t] = swx2;
    sLast[t] = key_value(k[15]);
  }
  __syncthreads();
  // total weight, the same in every wave: sum of 64 c over the blocks
  double wtot = 0.0;
  for (int b = lane; b < Ki / 64; b += 64) wtot += 64.0 * (double)sAbs[b];
  wtot += __shfl_xor(wtot, 32);
  wtot += __shfl_xor(wtot, 16);
  wtot = row16_sum(wtot);

  // ---- iterations ---------------------------------------------------------
  // Every wave keeps the whole state in lanes kk = lane & 15 (each 16-lane
  // row holds the same copy): level kk and threshold kk of the current
  // iteration. Every wave computes it from the same LDS values with the same
  // operations, so the copies agree bit for bit and so does the loop exit.
  const int kk = lane & 15;
  double Lc = (kk < nb) ? init.L[nbits - 1][kk] : 0.0;
  double Tc = (kk < nT) ? init.T[nbits - 1][kk] : 0.0;
  double prev = INFINITY;
  int it = 0, par = 0;
  const int g = t >> 4, e = t & 15;   // interval group, lane within it
  const uint64_t gmask = 0xFFFFull << (lane & 48);
  const int rowbase = lane & 48;
  bool go = max_iters > 0;
  while (go) {
    // thresholds in ascending order (a code counts thresholds below x, so
    // interval k lies between the k-th and (k+1)-th smallest threshold);
    // midpoints of increasing levels already are, else rank them
    const float T32 = __double2float_rd(Tc);
    float Ts = T32;
    const float Tup = __shfl(T32, rowbase | ((kk + 1) & 15));
    if (__ballot(kk + 1 < nT && !(T32 <= Tup)) != 0) {
      int rank = 0;
      for (int j = 0; j < nT; ++j) {
        const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(T32), j));
        rank += (v < T32 || (v == T32 && j < kk)) ? 1 : 0;
      }
      for (int j = 0; j < nT; ++j) {
        const int rj = __builtin_amdgcn_readlane(rank, j);
        const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(T32), j));
        if (rj == kk) Ts = vj;
      }
    }
    const float tlo = __shfl(Ts, (g - 1) & 15);
    const float thi = __shfl(Ts, g & 15);

    // interval g = positions [a, b)
    int a, b;
    sorted_positions<NT>(tlo, thi, sLast, sKey, e, gmask, a, b);
    if (g == 0) a = 0;
    if (g >= nT) b = Ki;
    if (g >= nb) { a = 0; b = 0; }
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    if (a < b) {
      const int sa = (a + 15) >> 4, sb = b >> 4;
      const int head_end = (sa <= sb) ? sa * 16 : b;
      const int tail_start = (sa <= sb) ? sb * 16 : b;
      const int p0 = a + e;
      if (p0 < head_end) {
        const uint64_t key = sKey[kslot(p0)];
        const double x = (double)key_value(key);
        const double w = (double)sAbs[(uint32_t)key >> 6];
        const double wx = w * x;
        s0 += w; s1 += wx; s2 += wx * x;
      }
      for (int q = sa + e; q < sb; q += 16) {
        s0 += sSeg[0][q]; s1 += sSeg[1][q]; s2 += sSeg[2][q];
      }
      const int p1 = tail_start + e;
      if (p1 < b) {
        const uint64_t key = sKey[kslot(p1)];
        const double x = (double)key_value(key);
        const double w = (double)sAbs[(uint32_t)key >> 6];
        const double wx = w * x;
        s0 += w; s1 += wx; s2 += wx * x;
      }
    }
    s0 = row16_sum(s0);
    s1 = row16_sum(s1);
    s2 = row16_sum(s2);
    if (g < nb && e == 0) {
      sBin[par][g][0] = s0;
      sBin[par][g][1] = s1;
      sBin[par][g][2] = s2;
    }
    __syncthreads();

    // levels, error, thresholds (every wave, lanes kk)
    double bw = 0.0, bwx = 0.0, bwx2 = 0.0;
    if (kk < nb) {
      bw = sBin[par][kk][0];
      bwx = sBin[par][kk][1];
      bwx2 = sBin[par][kk][2];
    }
    const double Ln = (bw > 0.0) ? bwx / bw : Lc;
    double sse = (kk < nb) ? (bwx2 - 2.0 * Ln * bwx + Ln * Ln * bw) : 0.0;
    sse = row16_sum(sse);
    const double mse = sse / wtot;
    Lc = Ln;
    const double Lup = __shfl(Lc, rowbase | ((kk + 1) & 15));
    Tc = (kk < nT) ? (Lc + Lup) / 2.0 : 0.0;
    ++it;
    const bool stop = mse >= prev;   // false while either is NaN, as in IEEE
    if (!stop) prev = mse;
    go = __builtin_amdgcn_readfirstlane((int)(!stop && it < max_iters)) != 0;
    par ^= 1;
  }

  // ---- outputs --------------------------------------------------------------
  const float l32 = (float)Lc;   // round to nearest even
  const float lnext = __shfl(l32, (lane & 48) | ((kk + 1) & 15));
  const float llast = __shfl(l32, nb - 1);
  if (t < 16) {
    levels[row * 16 + t] = (t < nb) ? l32 : llast;
    if (t < 15)
      thresholds[row * 15 + t] =
          (t < nT) ? __double2float_rd(((double)l32 + (double)lnext) / 2.0) : 3.0f;
    if (t == 0 && iterations) iterations[row] = it;
  }
}

template <int NT>
hipError_t launch_lloyd_nt(const void* W, int dtype, int64_t N, int64_t K, const uint8_t* row_bits,
                           int max_iters, const LloydInit& init, float* levels, float* thresholds,
                           int32_t* iterations, hipStream_t s) {
  const dim3 grid((unsigned)N), block(NT);
  if (dtype == LQ_F32)
    hipLaunchKernelGGL((k_lloyd<NT, float>), grid, block, 0, s, (const float*)W, K, row_bits,
                       max_iters, init, levels, thresholds, iterations);
  else if (dtype == LQ_BF16)
    hipLaunchKernelGGL((k_lloyd<NT, uint16_t>), grid, block, 0, s, (const uint16_t*)W, K, row_bits,
                       max_iters, init, levels, thresholds, iterations);
  else
    hipLaunchKernelGGL((k_lloyd<NT, _Float16>), grid, block, 0, s, (const _Float16*)W, K, row_bits,
                       max_iters, init, levels, thresholds, iterations);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lloyd(const void* W, int dtype, int64_t N, int64_t K, const uint8_t* row_bits,
                        int max_iters, float* levels, float* thresholds, int32_t* iterations,
                        hipStream_t s) {
  const LloydInit& init = lloyd_init();
  if (K <= 4096)
    return launch_lloyd_nt<256>(W, dtype, N, K, row_bits, max_iters, init, levels, thresholds, iterations, s);
  if (K <= 8192)
    return launch_lloyd_nt<512>(W, dtype, N, K, row_bits, max_iters, init, levels, thresholds, iterations, s);
  return launch_lloyd_nt<1024>(W, dtype, N, K, row_bits, max_iters, init, levels, thresholds, iterations, s);
}

}  // namespace lq
