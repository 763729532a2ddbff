// Codec kernels for gfx950: NF4 quantize, double quantization of the block
// constants, dequantization to bfloat16, and the per-channel codebook
// quantizer.
//
// QLoRA (Heng's Blog), "Contribution 1: 4-bit NormalFloat (NF4)": divide each
// block by its absmax, map to the nearest NF4 value, store 4-bit indices and
// the block constant. "Contribution 2: Double Quantization": FP32 constants per
// 64 weights, re-quantized with an 8-bit float at block size 256 after
// subtracting their mean. LowRA (cloud.tencent.com.cn), sections 3 and 4.1:
// per-output-channel quantization with custom thresholds and precision,
// groups of 64 scaled by absmax.
#include <float.h>

#include <algorithm>
#include <cmath>

#include "lq_device.h"

namespace lq {
namespace {

// ---------------------------------------------------------------------------
// NF4 quantize. A 64-weight block is 16 lanes x 4 consecutive weights (one
// 16-byte load per lane for float32 input). absmax is reduced inside the
// 16-lane DPP row. The code search uses the reciprocal of the block constant
// and a 33-bin table: bin j of x' = w * (1/c) holds at most one threshold, so
// code = base[j] + (x' > T[j]). Whenever x' lies within 2^-21 of that
// threshold -- closer than the float32 error of x' against the correctly
// rounded quotient w / c -- the quotient is computed exactly and used
// instead, so every code equals the one from IEEE division.
// ---------------------------------------------------------------------------
constexpr int kQuantPasses = 4;   // 16 blocks per pass per 256-thread WG

template <typename Tin> struct Load4;
template <> struct Load4<float> {
  __device__ static f32x4_t go(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
};
template <> struct Load4<uint16_t> {  // bfloat16 bits
  __device__ static f32x4_t go(const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return f32x4_t{bf16lo_to_f32(v.x), bf16hi_to_f32(v.x), bf16lo_to_f32(v.y), bf16hi_to_f32(v.y)};
  }
};
template <> struct Load4<_Float16> {
  __device__ static f32x4_t go(const _Float16* p) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = *reinterpret_cast<const h4*>(p);
    return f32x4_t{(float)v.x, (float)v.y, (float)v.z, (float)v.w};
  }
};

__device__ __forceinline__ uint32_t nf4_code(float w, float c, float r, bool fast_ok,
                                             const float* sT, const int32_t* sB) {
  const float xp = w * r;
  int j = (int)__builtin_fmaf(xp, 16.0f, 16.0f);
  j = min(max(j, 0), 32);
  const float T = sT[j];
  if (fast_ok && fabsf(xp - T) > 0x1p-21f) return (uint32_t)(sB[j] + (xp > T ? 1 : 0));
  const float x = (c > 0.0f) ? w / c : 0.0f;   // IEEE quotient
  int jj = (int)__builtin_fmaf(x, 16.0f, 16.0f);
  jj = min(max(jj, 0), 32);
  return (uint32_t)(sB[jj] + (x > sT[jj] ? 1 : 0));
}

template <typename Tin>
__global__ __launch_bounds__(256) void k_quantize_nf4(const Tin* __restrict__ W, int64_t n_blocks,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ absmax, Nf4Lut lut) {
  __shared__ float sT[33];
  __shared__ int32_t sB[33];
  if (threadIdx.x < 33) {
    sT[threadIdx.x] = lut.T[threadIdx.x];
    sB[threadIdx.x] = lut.base[threadIdx.x];
  }
  __syncthreads();
  const int i16 = threadIdx.x & 15;
  const int64_t blk0 = (int64_t)blockIdx.x * (16 * kQuantPasses) + (threadIdx.x >> 4);
  f32x4_t v[kQuantPasses];
#pragma unroll
  for (int p = 0; p < kQuantPasses; ++p) {
    const int64_t blk = blk0 + 16 * p;
    v[p] = (blk < n_blocks) ? Load4<Tin>::go(W + blk * 64 + i16 * 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int p = 0; p < kQuantPasses; ++p) {
    const int64_t blk = blk0 + 16 * p;
    float m = fmaxf(fmaxf(fabsf(v[p].x), fabsf(v[p].y)), fmaxf(fabsf(v[p].z), fabsf(v[p].w)));
    m = row16_max(m);
    const bool fast_ok = (m >= FLT_MIN) && (m <= 0x1p125f);
    const float r = fast_ok ? 1.0f / m : 0.0f;
    const uint32_t c0 = nf4_code(v[p].x, m, r, fast_ok, sT, sB);
    const uint32_t c1 = nf4_code(v[p].y, m, r, fast_ok, sT, sB);
    const uint32_t c2 = nf4_code(v[p].z, m, r, fast_ok, sT, sB);
    const uint32_t c3 = nf4_code(v[p].w, m, r, fast_ok, sT, sB);
    // two bytes per lane, element 4i in the high nibble of the first byte
    const uint32_t h = ((c0 << 4) | c1) | (((c2 << 4) | c3) << 8);
    const uint32_t d = h | (dpp_u32<DPP_QUAD_XOR1>(h) << 16);      // valid on even lanes
    const uint32_t d2 = dpp_u32<DPP_QUAD_XOR2>(d);                // lane 4k gets lane 4k+2's
    if (blk < n_blocks) {
      if ((i16 & 3) == 0)
        *reinterpret_cast<uint2*>(codes + blk * 32 + (i16 >> 2) * 8) = make_uint2(d, d2);
      if (i16 == 0) absmax[blk] = m;
    }
  }
}

// ---------------------------------------------------------------------------
// AQLoRA profiling pass (AQLoRA page, section 3.1): per layer, the mean
// squared error of the absmax-NF4 round trip and the fraction of weights with
// |w| < tau. Same block layout and code search as the quantizer; the
// reconstruction is the float32 product level * absmax, the error of each
// weight is squared in float64. Per workgroup: the error sum and the small
// count (both exact to float64 rounding of the sum), written to part[2 wg],
// then summed in a fixed order by k_profile_finish.
// ---------------------------------------------------------------------------
template <typename Tin>
__global__ __launch_bounds__(256) void k_profile_nf4(const Tin* __restrict__ W, int64_t n_blocks, Nf4Lut lut,
                                                     Nf4Levels lv, float tau_le, double* __restrict__ part) {
  __shared__ float sT[33];
  __shared__ int32_t sB[33];
  __shared__ float sQ[16];
  __shared__ double sW[2][4];
  if (threadIdx.x < 33) {
    sT[threadIdx.x] = lut.T[threadIdx.x];
    sB[threadIdx.x] = lut.base[threadIdx.x];
  }
  if (threadIdx.x < 16) sQ[threadIdx.x] = lv.q[threadIdx.x];
  __syncthreads();
  const int i16 = threadIdx.x & 15;
  const int64_t per_tile = 16 * kQuantPasses;
  const int64_t n_tiles = (n_blocks + per_tile - 1) / per_tile;
  double err = 0.0;
  uint32_t cnt = 0;
  // grid-stride over tiles of 64 blocks (fixed order for a given shape)
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t blk0 = tile * per_tile + (threadIdx.x >> 4);
    f32x4_t v[kQuantPasses];
#pragma unroll
    for (int p = 0; p < kQuantPasses; ++p) {
      const int64_t blk = blk0 + 16 * p;
      v[p] = (blk < n_blocks) ? Load4<Tin>::go(W + blk * 64 + i16 * 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int p = 0; p < kQuantPasses; ++p) {
      const int64_t blk = blk0 + 16 * p;
      float m = fmaxf(fmaxf(fabsf(v[p].x), fabsf(v[p].y)), fmaxf(fabsf(v[p].z), fabsf(v[p].w)));
      m = row16_max(m);
      const bool fast_ok = (m >= FLT_MIN) && (m <= 0x1p125f);
      const float r = fast_ok ? 1.0f / m : 0.0f;
      if (blk < n_blocks) {
        const float w4[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t code = nf4_code(w4[e], m, r, fast_ok, sT, sB);
          const float rec = sQ[code] * m;
          const double d = (double)w4[e] - (double)rec;   // exact
          err = __builtin_fma(d, d, err);
          cnt += (fabsf(w4[e]) <= tau_le) ? 1u : 0u;
        }
      }
    }
  }
  // fixed-order reductions: butterfly inside the wave, then the 4 waves in order
  double c = (double)cnt;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    err += __shfl_xor(err, off);
    c += __shfl_xor(c, off);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sW[0][wave] = err;
    sW[1][wave] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = ((sW[0][0] + sW[0][1]) + sW[0][2]) + sW[0][3];
    part[2 * blockIdx.x + 1] = ((sW[1][0] + sW[1][1]) + sW[1][2]) + sW[1][3];
  }
}

// One workgroup: thread t sums parts t, t + 1024, ... in order, then a
// pairwise tree over the 1024 thread sums. out = {err / n, count / n}.
__global__ __launch_bounds__(1024) void k_profile_finish(const double* __restrict__ part, int64_t nparts,
                                                         double n, double* __restrict__ out) {
  __shared__ double sE[1024], sC[1024];
  double e = 0.0, c = 0.0;
  for (int64_t i = threadIdx.x; i < nparts; i += 1024) {
    e += part[2 * i];
    c += part[2 * i + 1];
  }
  sE[threadIdx.x] = e;
  sC[threadIdx.x] = c;
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if ((int)threadIdx.x < h) {
      sE[threadIdx.x] += sE[threadIdx.x + h];
      sC[threadIdx.x] += sC[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = sE[0] / n;
    out[1] = sC[0] / n;
  }
}

// ---------------------------------------------------------------------------
// Double quantization. (1) per 256-constant block: float64 pairwise tree sum
// (4 leaves per lane, then a butterfly over the 64 lanes, which pairs
// neighbouring subtrees level by level). (2) pairwise tree over the block
// sums, 1024 leaves per workgroup, repeated until one value is left; zero
// padding to a power of two does not change the sum. (3) per block:
// d = c - mean, scale = max|d| / 448, code = E4M3(clamp(d / scale)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_dq_block_sums(const float* __restrict__ c, int64_t n_b,
                                                      double* __restrict__ sums) {
  const int l = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * 256 + 4 * l;
  double v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (base + i < n_b) ? (double)c[base + i] : 0.0;
  double s = (v[0] + v[1]) + (v[2] + v[3]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  if (l == 0) sums[blockIdx.x] = s;
}

__global__ __launch_bounds__(1024) void k_tree_reduce(const double* __restrict__ in, int64_t n_in,
                                                      double* __restrict__ out, int64_t n_b,
                                                      float* __restrict__ mean_out) {
  __shared__ double wsum[16];
  const int t = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * 1024 + t;
  double s = (i < n_in) ? in[i] : 0.0;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  if ((t & 63) == 0) wsum[t >> 6] = s;
  __syncthreads();
  if (t < 64) {
    double w = (t < 16) ? wsum[t] : 0.0;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) w = w + __shfl_xor(w, m);
    if (t == 0) {
      if (mean_out) *mean_out = (float)(w / (double)n_b);
      else out[blockIdx.x] = w;
    }
  }
}

// With SUMS, the block sums (at most 1024 of them) are passed instead of the
// mean, and every workgroup forms the mean itself by the same tree as
// k_tree_reduce: 1024 zero-padded leaves in order, 4 per lane summed in
// pairs, a butterfly over the 64 lanes, then the 4 wave sums in pairs, which
// is the same perfect binary tree, so every workgroup gets the same value;
// workgroup 0 stores it. This saves the launch of k_tree_reduce.
template <bool SUMS>
__global__ __launch_bounds__(256) void k_dq_encode(const float* __restrict__ c, int64_t n_b,
                                                   const double* __restrict__ sums, int64_t n_sums,
                                                   float* __restrict__ mean,
                                                   uint8_t* __restrict__ absmax_q,
                                                   float* __restrict__ dq_scale) {
  __shared__ float wmax[4];
  __shared__ double wsum[4];
  const int t = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * 256 + t;
  const float cj = (j < n_b) ? c[j] : 0.0f;
  float mu;
  if constexpr (SUMS) {
    double v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (4 * t + i < n_sums) ? sums[4 * t + i] : 0.0;
    double w = (v[0] + v[1]) + (v[2] + v[3]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) w = w + __shfl_xor(w, m);
    if ((t & 63) == 0) wsum[t >> 6] = w;
    __syncthreads();
    const double total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    mu = (float)(total / (double)n_b);
    if (blockIdx.x == 0 && t == 0) *mean = mu;
  } else {
    mu = *mean;
  }
  const float d = (j < n_b) ? cj - mu : 0.0f;
  float a = wave_max(fabsf(d));
  if ((t & 63) == 0) wmax[t >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s2 = a / 448.0f;
  if (t == 0) dq_scale[blockIdx.x] = s2;
  uint32_t code = 0;
  if (s2 > 0.0f) {
    float v = d / s2;
    v = fminf(fmaxf(v, -448.0f), 448.0f);
    code = e4m3_encode(v);
  }
  if (j < n_b) absmax_q[j] = (uint8_t)code;
}

// ---------------------------------------------------------------------------
// Dequant to bfloat16. A wave covers 2048 consecutive elements in 4 passes;
// in pass d lane l handles elements 512d + 8l .. +7 (one dword of codes), so
// each code load reads 256 contiguous bytes and each 16-byte store instruction
// writes 1 KB contiguous. NF4: a 256-entry table in LDS maps a code byte to
// its two float32 levels.
// ---------------------------------------------------------------------------
template <bool DQ>
__global__ __launch_bounds__(256) void k_dequant_nf4(const uint8_t* __restrict__ codes, QConst qc,
                                                     int64_t n, uint16_t* __restrict__ out,
                                                     Nf4Levels lv) {
  __shared__ f32x2_t pair[256];
  pair[threadIdx.x] = f32x2_t{lv.q[threadIdx.x >> 4], lv.q[threadIdx.x & 15]};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t e_base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2048 + 8 * lane;
  const float mean = DQ ? *qc.dq_mean : 0.0f;
  uint32_t w[4];
  float c0[4], s2[4];
  uint32_t q8[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int64_t e = min(e_base + 512 * d, n - 8);   // n % 64 == 0; clamped lanes do not store
    w[d] = *reinterpret_cast<const uint32_t*>(codes + e / 2);
    const int64_t blk = e >> 6;
    if (DQ) {
      q8[d] = qc.absmax_q[blk];
      s2[d] = qc.dq_scale[blk >> 8];
    } else {
      c0[d] = qc.absmax[blk];
    }
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int64_t e = e_base + 512 * d;
    const float cp = DQ ? __builtin_fmaf(e4m3_decode(q8[d]), s2[d], mean) : c0[d];
    u32x4_t o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x2_t q = pair[(w[d] >> (8 * b)) & 0xFFu];
      o[b] = pack_bf16x2(q.x * cp, q.y * cp);
    }
    if (e < n) *reinterpret_cast<u32x4_t*>(out + e) = o;
  }
}

// Codebook dequant: one thread per 8 elements of a 64-block (one byte of
// each bit-plane). Row i's levels live in levels[i*16 ...].
__global__ __launch_bounds__(256) void k_dequant_codebook(const uint8_t* __restrict__ codes,
                                                          QConst qc, int64_t N, int64_t K,
                                                          const uint8_t* __restrict__ row_bits,
                                                          const int64_t* __restrict__ row_offset,
                                                          const float* __restrict__ levels,
                                                          uint16_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;   // group of 8 elements
  const int64_t groups_per_row = K / 8;
  if (g >= N * groups_per_row) return;
  const int64_t row = g / groups_per_row;
  const int64_t k8 = g - row * groups_per_row;                 // 8-element group in row
  const int64_t blk_in_row = k8 >> 3;
  const int byte_in_plane = (int)(k8 & 7);
  const int nb = min(max((int)row_bits[row], 1), 4);
  const uint8_t* src = codes + row_offset[row] + blk_in_row * 8 * nb;
  uint32_t code[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int p = 0; p < nb; ++p) {
    const uint32_t byte = src[8 * p + byte_in_plane];
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e] |= ((byte >> e) & 1u) << p;
  }
  const float cp = block_const(qc, row * (K / 64) + blk_in_row);
  const float* L = levels + row * 16;
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(L[code[2 * e]] * cp, L[code[2 * e + 1]] * cp);
  *reinterpret_cast<u32x4_t*>(out + row * K + k8 * 8) = o;
}

// ---------------------------------------------------------------------------
// Codebook quantize: one workgroup per row. Each wave takes 256-element
// chunks of the row (four 64-blocks); lane l holds elements 4(l & 15) ..
// 4(l & 15) + 3 of block l >> 4, so a block is one 16-lane DPP row and its
// absmax is a row maximum. x = w / c is the IEEE quotient; the code is the
// number of the row's thresholds strictly below x. Bit-plane p of a block is
// assembled as two 32-bit words, each the OR over 8 lanes of their 4-bit
// slices.
// ---------------------------------------------------------------------------
template <typename Tin, bool VEC>
__device__ __forceinline__ void load4(const Tin* p, float (&w)[4]);
template <> __device__ __forceinline__ void load4<float, true>(const float* p, float (&w)[4]) {
  const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
  w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
}
template <> __device__ __forceinline__ void load4<float, false>(const float* p, float (&w)[4]) {
  w[0] = p[0]; w[1] = p[1]; w[2] = p[2]; w[3] = p[3];
}
template <> __device__ __forceinline__ void load4<uint16_t, true>(const uint16_t* p, float (&w)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  w[0] = bf16lo_to_f32(v.x); w[1] = bf16hi_to_f32(v.x); w[2] = bf16lo_to_f32(v.y); w[3] = bf16hi_to_f32(v.y);
}
template <> __device__ __forceinline__ void load4<uint16_t, false>(const uint16_t* p, float (&w)[4]) {
  for (int j = 0; j < 4; ++j) w[j] = bf16_to_f32(p[j]);
}
template <> __device__ __forceinline__ void load4<_Float16, true>(const _Float16* p, float (&w)[4]) {
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  const h4_t v = *reinterpret_cast<const h4_t*>(p);
  w[0] = (float)v[0]; w[1] = (float)v[1]; w[2] = (float)v[2]; w[3] = (float)v[3];
}
template <> __device__ __forceinline__ void load4<_Float16, false>(const _Float16* p, float (&w)[4]) {
  for (int j = 0; j < 4; ++j) w[j] = (float)p[j];
}

__device__ __forceinline__ uint32_t row8_or(uint32_t v) {
  v |= dpp_u32<DPP_QUAD_XOR1>(v);
  v |= dpp_u32<DPP_QUAD_XOR2>(v);
  v |= dpp_u32<DPP_ROW_HALF_MIRROR>(v);
  return v;
}

// One row at a compile-time width: thresholds in registers, the wave's
// chunks of the row loaded together before any is processed.
template <int NBITS, typename Tin, bool VEC>
__device__ __forceinline__ void codebook_row(const Tin* __restrict__ Wr, int64_t blocks,
                                             const float* __restrict__ Tr, uint8_t* __restrict__ dst,
                                             float* __restrict__ absmax_row, int wave, int lane) {
  constexpr int NT = (1 << NBITS) - 1;
  constexpr int BATCH = 4;
  float tr[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) tr[k] = Tr[k];
  const int g = lane >> 4, m = lane & 15;
  for (int64_t c0 = wave; c0 * 4 < blocks; c0 += 4 * BATCH) {
    float w[BATCH][4];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int64_t blk = (c0 + 4 * b) * 4 + g;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[b][j] = 0.0f;
      if (blk < blocks) load4<Tin, VEC>(Wr + blk * 64 + 4 * m, w[b]);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int64_t blk = (c0 + 4 * b) * 4 + g;
      const bool live = blk < blocks;   // uniform over the 16-lane row
      float mx = fmaxf(fmaxf(fabsf(w[b][0]), fabsf(w[b][1])), fmaxf(fabsf(w[b][2]), fabsf(w[b][3])));
      mx = row16_max(mx);
      uint32_t code[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = (mx > 0.0f) ? w[b][j] / mx : 0.0f;
        uint32_t cj = 0;
#pragma unroll
        for (int k = 0; k < NT; ++k) cj += (x > tr[k]) ? 1u : 0u;
        code[j] = cj;
      }
#pragma unroll
      for (int p = 0; p < NBITS; ++p) {
        uint32_t nib = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) nib |= ((code[j] >> p) & 1u) << j;
        const uint32_t word = row8_or(nib << (4 * (m & 7)));
        if (live && (m & 7) == 0)
          *reinterpret_cast<uint32_t*>(dst + blk * 8 * NBITS + 8 * p + 4 * (m >> 3)) = word;
      }
      if (live && m == 0) absmax_row[blk] = mx;
    }
  }
}

template <typename Tin, bool VEC>
__global__ __launch_bounds__(256) void k_quantize_codebook(const Tin* __restrict__ W, int64_t K,
                                                           const uint8_t* __restrict__ row_bits,
                                                           const int64_t* __restrict__ row_offset,
                                                           const float* __restrict__ T,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int nb = min(max((int)row_bits[row], 1), 4);
  const int64_t blocks = K / 64;
  const Tin* Wr = W + row * K;
  const float* Tr = T + row * 15;
  uint8_t* dst = codes + row_offset[row];
  float* am = absmax + row * blocks;
  switch (nb) {
    case 1: codebook_row<1, Tin, VEC>(Wr, blocks, Tr, dst, am, wave, lane); break;
    case 2: codebook_row<2, Tin, VEC>(Wr, blocks, Tr, dst, am, wave, lane); break;
    case 3: codebook_row<3, Tin, VEC>(Wr, blocks, Tr, dst, am, wave, lane); break;
    default: codebook_row<4, Tin, VEC>(Wr, blocks, Tr, dst, am, wave, lane); break;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quantize_nf4(const void* W, int dtype, int64_t n_blocks, uint8_t* codes,
                               float* absmax, hipStream_t s) {
  const int64_t per_wg = 16 * kQuantPasses;
  const dim3 grid((unsigned)((n_blocks + per_wg - 1) / per_wg));
  const Nf4Lut& lut = tables().lut;
  if (dtype == LQ_F32)
    hipLaunchKernelGGL(k_quantize_nf4<float>, grid, dim3(256), 0, s, (const float*)W, n_blocks, codes, absmax, lut);
  else if (dtype == LQ_BF16)
    hipLaunchKernelGGL(k_quantize_nf4<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)W, n_blocks, codes, absmax, lut);
  else
    hipLaunchKernelGGL(k_quantize_nf4<_Float16>, grid, dim3(256), 0, s, (const _Float16*)W, n_blocks, codes, absmax, lut);
  return hipGetLastError();
}

static int64_t profile_grid(int64_t n_blocks) {
  const int64_t per_tile = 16 * kQuantPasses;
  const int64_t n_tiles = (n_blocks + per_tile - 1) / per_tile;
  return std::min<int64_t>(n_tiles, 2048);   // 8 workgroups of 4 waves per CU
}

size_t profile_ws_doubles(int64_t n_blocks) { return (size_t)(2 * profile_grid(n_blocks)); }

hipError_t launch_profile_nf4(const void* W, int dtype, int64_t n_blocks, double tau, double* stats,
                              double* ws, hipStream_t s) {
  const int64_t nwg = profile_grid(n_blocks);
  const dim3 grid((unsigned)nwg);
  const Nf4Lut& lut = tables().lut;
  const Nf4Levels& lv = tables().lv;
  // |w| < tau for a float32 |w|  <=>  |w| <= the largest float32 below tau
  float tau_le = (float)tau;
  if ((double)tau_le >= tau) tau_le = std::nextafter(tau_le, 0.0f);
  if (dtype == LQ_F32)
    hipLaunchKernelGGL(k_profile_nf4<float>, grid, dim3(256), 0, s, (const float*)W, n_blocks, lut, lv, tau_le, ws);
  else if (dtype == LQ_BF16)
    hipLaunchKernelGGL(k_profile_nf4<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)W, n_blocks, lut, lv, tau_le, ws);
  else
    hipLaunchKernelGGL(k_profile_nf4<_Float16>, grid, dim3(256), 0, s, (const _Float16*)W, n_blocks, lut, lv, tau_le, ws);
  hipLaunchKernelGGL(k_profile_finish, dim3(1), dim3(1024), 0, s, ws, nwg, (double)n_blocks * 64.0, stats);
  return hipGetLastError();
}

size_t double_quant_ws_doubles(int64_t n_blocks) {
  const int64_t n_d = (n_blocks + 255) / 256;
  int64_t total = n_d, level = n_d;
  while (level > 1024) {
    level = (level + 1023) / 1024;
    total += level;
  }
  return (size_t)total + 16;
}

hipError_t launch_double_quant(const float* absmax, int64_t n_b, uint8_t* absmax_q,
                               float* dq_scale, float* dq_mean, double* ws, hipStream_t s) {
  const int64_t n_d = (n_b + 255) / 256;
  hipLaunchKernelGGL(k_dq_block_sums, dim3((unsigned)n_d), dim3(64), 0, s, absmax, n_b, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_d <= 1024) {   // one level of the tree: the encoder forms the mean itself
    hipLaunchKernelGGL(k_dq_encode<true>, dim3((unsigned)n_d), dim3(256), 0, s, absmax, n_b,
                       (const double*)ws, n_d, dq_mean, absmax_q, dq_scale);
    return hipGetLastError();
  }
  double* cur = ws;
  int64_t n = n_d;
  while (n > 1024) {
    const int64_t groups = (n + 1023) / 1024;
    double* nxt = cur + n;
    hipLaunchKernelGGL(k_tree_reduce, dim3((unsigned)groups), dim3(1024), 0, s, cur, n, nxt, n_b,
                       (float*)nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    cur = nxt;
    n = groups;
  }
  hipLaunchKernelGGL(k_tree_reduce, dim3(1), dim3(1024), 0, s, cur, n, (double*)nullptr, n_b, dq_mean);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_dq_encode<false>, dim3((unsigned)n_d), dim3(256), 0, s, absmax, n_b,
                     (const double*)nullptr, (int64_t)0, dq_mean, absmax_q, dq_scale);
  return hipGetLastError();
}

hipError_t launch_dequant(const QWeight& w, uint16_t* out, hipStream_t s) {
  if (w.format == LQ_FMT_NF4) {
    const int64_t n = w.N * w.K;
    const dim3 grid((unsigned)((n + 8191) / 8192));
    if (w.qc.absmax) hipLaunchKernelGGL(k_dequant_nf4<false>, grid, dim3(256), 0, s, w.codes, w.qc, n, out, tables().lv);
    else hipLaunchKernelGGL(k_dequant_nf4<true>, grid, dim3(256), 0, s, w.codes, w.qc, n, out, tables().lv);
  } else {
    const int64_t n_groups = w.N * w.K / 8;
    hipLaunchKernelGGL(k_dequant_codebook, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0,
                       s, w.codes, w.qc, w.N, w.K, w.row_bits, w.row_offset, w.levels, out);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_codebook(const void* W, int dtype, int64_t N, int64_t K,
                                    const uint8_t* row_bits, const int64_t* row_offset,
                                    const float* T, uint8_t* codes, float* absmax, hipStream_t s) {
  const dim3 grid((unsigned)N), block(256);
  const uintptr_t a = (uintptr_t)W;
  if (dtype == LQ_F32) {
    if (a % 16 == 0)
      hipLaunchKernelGGL((k_quantize_codebook<float, true>), grid, block, 0, s, (const float*)W, K, row_bits, row_offset, T, codes, absmax);
    else
      hipLaunchKernelGGL((k_quantize_codebook<float, false>), grid, block, 0, s, (const float*)W, K, row_bits, row_offset, T, codes, absmax);
  } else if (dtype == LQ_BF16) {
    if (a % 8 == 0)
      hipLaunchKernelGGL((k_quantize_codebook<uint16_t, true>), grid, block, 0, s, (const uint16_t*)W, K, row_bits, row_offset, T, codes, absmax);
    else
      hipLaunchKernelGGL((k_quantize_codebook<uint16_t, false>), grid, block, 0, s, (const uint16_t*)W, K, row_bits, row_offset, T, codes, absmax);
  } else {
    if (a % 8 == 0)
      hipLaunchKernelGGL((k_quantize_codebook<_Float16, true>), grid, block, 0, s, (const _Float16*)W, K, row_bits, row_offset, T, codes, absmax);
    else
      hipLaunchKernelGGL((k_quantize_codebook<_Float16, false>), grid, block, 0, s, (const _Float16*)W, K, row_bits, row_offset, T, codes, absmax);
  }
  return hipGetLastError();
}

}  // namespace lq
