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

// Four packed FP4 bytes (8 nibbles, element 2j in the low nibble of byte j)
// -> 8 fp16 values E2M1 * scale.  The hardware converts each byte into two
// fp16 (low nibble first) with a unit scale; the per-block E4M3 factor is then
// applied with one packed fp16 multiply per pair, exact by the argument above.
__device__ __forceinline__ f16x8 dequant8(uint32_t packed, f16x2 scale2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3);
  p0 *= scale2;
  p1 *= scale2;
  p2 *= scale2;
  p3 *= scale2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ f16x2 scale_f16x2(uint32_t byte) {
  _Float16 h = (_Float16)e4m3_to_f32(byte);
  f16x2 r = {h, h};
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
