// NVFP4 weights to bf16 MFMA operands, shared by the decode and prefill
// kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {
namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Value of an E4M3 block-scale byte (non-negative, not NaN: checked on the
// host) as fp32, from its fields: exponent bits 6..3 (bias 7), mantissa
// bits 2..0, subnormal m * 2^-9.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// 8 E2M1 codes times an E4M3 block scale s -> 8 bf16, exactly.  The convert
// to fp32 applies s's power of two (it reads only the exponent field); s's
// significand (1 + m/8, or 0 for a zero scale) multiplies in fp32.  Every
// product has at most 6 significant bits, so it is exact in fp32 and in
// bf16, and one byte permute packs the top halves of two products.
__device__ __forceinline__ bf16x8 dequant8_nv(uint32_t q, uint32_t sbyte) {
  const float s = e4m3_value(sbyte);
  const float f = s == 0.0f ? 0.0f : __uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
  auto pair = [f](f32x2 v) {
    return __builtin_amdgcn_perm(__float_as_uint(v[1] * f), __float_as_uint(v[0] * f), 0x07060302u);
  };
  u32x4 r;
  r[0] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 0));
  r[1] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 1));
  r[2] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 2));
  r[3] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 3));
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace nvfp4
}  // namespace moe
