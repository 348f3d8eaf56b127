// Device-side helpers shared by the NVFP4 kernels (gfx950 only).
//
// Number formats (kernelindex "NVFP4 linear layer", description: FP4 operands
// with FP8 E4M3FN scales, one per 16 elements):
//   E2M1 nibble : bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa;
//                 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
//   E4M3FN byte : bit 7 sign, bits 6-3 exponent (bias 7), bits 2-0 mantissa,
//                 exponent 0 subnormal, 0x7F/0xFF NaN, largest finite 448.
// Any E2M1 value times any finite E4M3 value has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16: dequantising to fp16
// and multiplying on the matrix cores with fp32 accumulation forms every
// product x_k * w_k exactly; only the fp32 sums round.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// E4M3FN byte -> fp32 (hardware OCP FP8 conversion; exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// {S, S} as fp16 bits with S = E4M3(byte) * 2^-8: E4M3 and fp16 share the
// subnormal/normal structure, so the 7 magnitude bits shifted left by 7 are
// exactly E4M3 * 2^-8 in fp16 (possibly subnormal); the sign moves to bit 15.
// The factor 2^8 is restored by converting nibbles with a scale of 256.
__device__ __forceinline__ uint32_t scale_pair_bits(uint32_t byte) {
  const uint32_t h = ((byte & 0x7Fu) << 7) | ((byte & 0x80u) << 8);
  return h | (h << 16);
}

__device__ __forceinline__ f16x8 dequant8_scaled(uint32_t packed, uint32_t pair_bits) {
  f16x2 s2;
  __builtin_memcpy(&s2, &pair_bits, 4);
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 3);
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Output writer: dtype 0 = fp32, 1 = bf16.
__device__ __forceinline__ void store_out(void* y, int64_t idx, float v, int dtype) {
  if (dtype == 0)
    reinterpret_cast<float*>(y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(v);
}

}  // namespace nvfp4
