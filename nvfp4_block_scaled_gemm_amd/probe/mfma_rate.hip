// Measurement probe (not part of the GEMM library): the sustained rate of
// v_mfma_f32_32x32x16_f16 on gfx950, alone and with NV independent vector
// instructions issued after each MFMA -- the same two instructions that
// dequantise NVFP4 operands in the GEMM (FP4 -> fp16 conversion and packed
// fp16 multiply), alternating.  Each wave runs four independent accumulator
// chains, held in AGPRs as in the GEMM, so the matrix core never waits on a
// result; the vector instructions work on registers the MFMAs do not touch.
//
//   int probe_mfma_rate(int nv, int blocks, int threads, int iters, float* out, void* stream)
//
// launches `blocks` workgroups of `threads` threads (a multiple of 64, at
// most 1024); each wave issues 4 * iters MFMAs.  `out` must hold
// blocks * threads floats (device memory; a checksum that keeps the work
// live).  Returns 0, -1 for an unsupported nv or shape, or the HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int NV>
__global__ __launch_bounds__(1024) void mfma_rate_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  f16x8 a[4], b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = (_Float16)(0.001f * (float)(tid + j));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) a[i][j] = (_Float16)(0.002f * (float)(tid * i + j));
  f32x16 acc[4] = {};
  uint32_t u[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) u[c] = 0x3c003c00u + (uint32_t)(c + tid);
  const uint32_t mul = 0x3c013bffu + (uint32_t)(tid & 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // accumulators in AGPRs, as in the GEMM (the "a" constraint)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(a[i]), "v"(b));
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int c = (i * NV + v) & 7;
        if (v & 1)
          asm volatile("v_pk_mul_f16 %0, %0, %1" : "+v"(u[c]) : "v"(mul));
        else
          asm volatile("v_cvt_scalef32_pk_f16_fp4 %0, %0, 1.0" : "+v"(u[c]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
#pragma unroll
  for (int c = 0; c < 8; ++c) s += (float)(u[c] & 0xffu);
  out[(int64_t)blockIdx.x * blockDim.x + tid] = s;
}

template <int NV>
int launch(int blocks, int threads, int iters, float* out, hipStream_t stream) {
  mfma_rate_kernel<NV><<<blocks, threads, 0, stream>>>(out, iters);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" int probe_mfma_rate(int nv, int blocks, int threads, int iters, float* out,
                               void* stream) {
  if (blocks <= 0 || threads <= 0 || threads > 1024 || threads % 64 != 0 || iters < 0 ||
      out == nullptr)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  switch (nv) {
    case 0: return launch<0>(blocks, threads, iters, out, s);
    case 2: return launch<2>(blocks, threads, iters, out, s);
    case 4: return launch<4>(blocks, threads, iters, out, s);
    case 6: return launch<6>(blocks, threads, iters, out, s);
    case 8: return launch<8>(blocks, threads, iters, out, s);
    default: return -1;
  }
}
