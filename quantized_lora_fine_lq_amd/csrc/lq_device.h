// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, DPP cross-lane operations, the OCP E4M3 codec and the
// block-constant decoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lq_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace lq {

// Two float32 -> packed bfloat16x2 (round to nearest even; v_cvt_pk_bf16_f32).
// `lo` lands in bits 15..0, i.e. at the lower address.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// DPP permutes (all lanes valid for these controls).
enum : int {
  DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_MIRROR = 0x140,
};
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// max over the 16 lanes of a DPP row
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f32<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f32<DPP_ROW_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ---- OCP E4M3 (bias 7, max 448, subnormal step 2^-9) ------------------------
// Placing the 7 magnitude bits at float32 bit 20 gives 2^(e-127) (1 + m/8)
// for e > 0 and the float32 denormal m 2^-129 for e = 0; scaling by 2^120 is
// exact and yields 2^(e-7) (1 + m/8) and m 2^-9 respectively.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __uint_as_float(((code & 0x7Fu) << 20) | ((code & 0x80u) << 24)) * 0x1p120f;
}

// v must be finite and within [-448, 448]. Round to nearest, ties to even.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {                  // |v| < 2^-6: steps of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 127u;  // -6 .. 8 (mod 2^32)
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t q = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    code = ((e + 7u) << 3) + q;           // q == 8 carries into the exponent
  }
  return code | sign;
}

// Block constant j of a quantized weight: float32, or decoded double quant.
__device__ __forceinline__ float block_const(const QConst& qc, int64_t j) {
  if (qc.absmax) return qc.absmax[j];
  const float e = e4m3_decode(qc.absmax_q[j]);
  return __builtin_fmaf(e, qc.dq_scale[j >> 8], *qc.dq_mean);
}

}  // namespace lq
