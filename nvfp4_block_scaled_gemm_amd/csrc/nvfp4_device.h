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

#include <type_traits>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// E4M3FN byte -> fp32 (hardware OCP FP8 conversion; exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// The four E4M3 scale bytes of a lane's 64 K-elements as two fp16 pairs
// (blocks 0,1 and 2,3), from the hardware FP8 pair conversion (exact: every
// E4M3 value is an fp16 value).
struct Scales {
  f16x2 s01, s23;
};

__device__ __forceinline__ Scales to_scales(uint32_t s4) {
  return {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, false),
          __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, true)};
}

// Elements 4H .. 4H+3 of MFMA step T: a lane holds 64 consecutive K-elements
// as 8 packed dwords (step T uses dword T, i.e. block T/2 of the lane).  The
// hardware converts each byte into two fp16 (low nibble first, unit scale)
// and one packed multiply per pair applies the block's E4M3 scale (the
// selected half broadcast to both lanes).
template <int T, int H>
__device__ __forceinline__ void dequant_piece(uint32_t w, const Scales& sc, f16x8& out) {
  const f16x2 s = ((T >> 1) < 2) ? sc.s01 : sc.s23;
  constexpr int HALF = (T >> 1) & 1;
  const f16x2 s2 = __builtin_shufflevector(s, s, HALF, HALF);
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2 * H) * s2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2 * H + 1) * s2;
  out[4 * H + 0] = p0[0];
  out[4 * H + 1] = p0[1];
  out[4 * H + 2] = p1[0];
  out[4 * H + 3] = p1[1];
}

template <int T>
__device__ __forceinline__ f16x8 dequant_step(uint32_t w, const Scales& sc) {
  f16x8 out;
  dequant_piece<T, 0>(w, sc, out);
  dequant_piece<T, 1>(w, sc, out);
  return out;
}

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// 2 * E2M1 magnitude of code c = 0..7 is 0,1,2,3,4,6,8,12: one hex digit each
// of 0xC8643210, read at digit c; bit 3 of the nibble is the sign.
__device__ __forceinline__ int e2m1_x2(uint32_t nib) {
  const int mag = (int)((0xC8643210u >> (4u * (nib & 7u))) & 15u);
  return (nib & 8u) ? -mag : mag;
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
