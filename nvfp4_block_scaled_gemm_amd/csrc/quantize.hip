// NVFP4 quantiser: x (fp32 | bf16) [rows, cols] -> packed E2M1 nibbles,
// E4M3FN block scales (one per 16 elements) and an fp32 global scale.
//
// Format: kernelindex "NVFP4 linear layer" (description: FP4 values with FP8
// E4M3FN scales per 16 elements); magik.net "The 3.7 PFLOPS Revelation",
// "Input Knowledge" item 2 (two values per byte, K//2 data, K//16 scales).
// Quantisation runs ahead of the GEMM and is timed apart (leverageai
// "blackwell-nvfp4-gemm-optimization", "What is this?").
//
// Semantics (the pages leave them open; the reading taken is that every
// stored quantity is rounded once from its exact real value):
//   g      = fl32(amax_t / 2688)
//   s_b    = nearest E4M3 (ties to even code, saturating at 448) to amax_b/(6g)
//   code_i = nearest E2M1 magnitude (ties to even, saturating at 6) to
//            |x_i| / (E4M3(s_b) * g); 0 when s_b == 0
//   nibble = signbit(x_i) << 3 | code_i
// All decisions are exact comparisons of the input against products of a
// few-bit midpoint and g, which are exact in fp64 (at most 31 significant
// bits), or against their fp32 neighbours chosen to give the same answer.
//
// Two kernels: an amax pass writing one partial maximum per workgroup, and an
// encode pass in which every workgroup reduces the partials (deterministic,
// no atomics, no memset), derives g, and encodes its 16-element blocks.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

// ---- loading one 16-element block as |x| bit patterns and sign bits -------

struct Block16 {
  float a[16];      // |x_i| as fp32 (exact for both input types)
  uint32_t sign;    // bit i = signbit(x_i)
};

__device__ __forceinline__ void load_block(const void* x, int dtype, int64_t elem_off,
                                           Block16& b) {
  b.sign = 0;
  if (dtype == 1) {  // bf16: two 16-byte loads
    const u32x4* p = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(x) + elem_off);
    u32x4 v0 = p[0], v1 = p[1];
    uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lo = w[i] << 16, hi = w[i] & 0xFFFF0000u;
      b.sign |= (lo >> 31) << (2 * i);
      b.sign |= (hi >> 31) << (2 * i + 1);
      b.a[2 * i] = __uint_as_float(lo & 0x7FFFFFFFu);
      b.a[2 * i + 1] = __uint_as_float(hi & 0x7FFFFFFFu);
    }
  } else {  // fp32: four 16-byte loads
    const u32x4* p = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const float*>(x) + elem_off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = p[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b.sign |= (v[i] >> 31) << (4 * j + i);
        b.a[4 * j + i] = __uint_as_float(v[i] & 0x7FFFFFFFu);
      }
    }
  }
}

__device__ __forceinline__ uint32_t block_amax_bits(const Block16& b) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(b.a[i]));
  return m;  // non-negative floats order like their bit patterns
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* lds) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = max(r, lds[w]);
  __syncthreads();
  return r;
}

// ---- amax pass ------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void amax_kernel(const void* __restrict__ x, int dtype,
                                                        int64_t rows, int64_t nblk_row,
                                                        int64_t ld_x, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t total = rows * nblk_row;
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * kThreads) {
    const int64_t r = c / nblk_row, j = c - r * nblk_row;
    Block16 b;
    load_block(x, dtype, r * ld_x + j * 16, b);
    m = max(m, block_amax_bits(b));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// ---- encode pass ----------------------------------------------------------

// Midpoint between E4M3 codes c and c+1 (c in 0..125) times 6, exactly:
// (E >= 1 ? 16 : 0) + 2m + 1 over 2^(11 - max(E,1)), E = c >> 3, m = c & 7.
__device__ __forceinline__ double e4m3_mid_times6(int c) {
  const int e = c >> 3, m = c & 7;
  const int mant = (e >= 1 ? 16 : 0) + 2 * m + 1;
  const int ex = (e >= 1 ? e : 1) - 11;
  return __builtin_ldexp((double)(6 * mant), ex);
}

// Exact value of E4M3 code c in 0..126.
__device__ __forceinline__ double e4m3_value(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? __builtin_ldexp((double)m, -9) : __builtin_ldexp((double)(8 + m), e - 10);
}

// Neighbours of a finite non-negative fp32 (bit pattern +-1; 0 steps up to
// the smallest subnormal).
__device__ __forceinline__ float next_up(float f) { return __uint_as_float(__float_as_uint(f) + 1u); }
__device__ __forceinline__ float next_down(float f) { return __uint_as_float(__float_as_uint(f) - 1u); }

// Largest fp32 <= t and smallest fp32 >= t, for finite non-negative t.
__device__ __forceinline__ float round_down_f32(double t) {
  float f = (float)t;
  if ((double)f > t) f = next_down(f);
  return f;
}
__device__ __forceinline__ float round_up_f32(double t) {
  float f = (float)t;
  if ((double)f < t) f = next_up(f);
  return f;
}

__global__ __launch_bounds__(kThreads) void encode_kernel(
    const void* __restrict__ x, int dtype, int64_t rows, int64_t nblk_row, int64_t ld_x,
    uint8_t* __restrict__ q, uint8_t* __restrict__ s, float* __restrict__ gscale,
    const uint32_t* __restrict__ partial, int npartial, int scale_given) {
  __shared__ uint32_t red[kThreads / 64];
  float g;
  if (scale_given) {
    g = *gscale;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
    m = block_max(m, red);
    // fl32(amax / 2688): the fp64 quotient rounds to the same fp32 as the
    // exact one, since amax / 2688 can come no closer to an fp32 rounding
    // boundary than 2^-25 / 21 relative unless it lies on it exactly.
    g = (float)((double)__uint_as_float(m) / 2688.0);
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = g;
  }
  const double gd = (double)g;
  // E2M1 midpoints between magnitude codes j and j+1.
  const double mid2[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};

  const int64_t total = rows * nblk_row;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * kThreads) {
    const int64_t r = c / nblk_row, j = c - r * nblk_row;
    Block16 b;
    load_block(x, dtype, r * ld_x + j * 16, b);
    const double amax_b = (double)__uint_as_float(block_amax_bits(b));

    // Scale code: number of midpoints c (0..125) the quotient amax_b/(6g) lies
    // above, a tie moving up only from an odd c (so the result is even).
    int code_s = 0;
    if (gd > 0.0) {
      int lo = 0, hi = 126;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const double t = e4m3_mid_times6(mid) * gd;   // exact
        const bool up = amax_b > t || (amax_b == t && (mid & 1));
        if (up) lo = mid + 1; else hi = mid;
      }
      code_s = lo;
    }

    uint32_t lo_word = 0, hi_word = 0;
    if (code_s != 0) {
      const double S = e4m3_value(code_s) * gd;         // exact
      // fp32 thresholds V_j such that code_i = #{ j : |x_i| >= V_j }:
      // odd j (tie rounds up): smallest fp32 >= mid_j*S;
      // even j (tie stays):    the fp32 just above the largest fp32 <= mid_j*S.
      float V[7];
#pragma unroll
      for (int t = 0; t < 7; ++t) {
        const double u = mid2[t] * S;                     // exact
        V[t] = (t & 1) ? round_up_f32(u)
                       : next_up(round_down_f32(u));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t code = 0;
#pragma unroll
        for (int t = 0; t < 7; ++t) code += (b.a[i] >= V[t]) ? 1u : 0u;
        const uint32_t nib = code | (((b.sign >> i) & 1u) << 3);
        if (i < 8) lo_word |= nib << (4 * i);
        else hi_word |= nib << (4 * (i - 8));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t nib = ((b.sign >> i) & 1u) << 3;
        if (i < 8) lo_word |= nib << (4 * i);
        else hi_word |= nib << (4 * (i - 8));
      }
    }
    u32x2 packed = {lo_word, hi_word};
    *reinterpret_cast<u32x2*>(q + r * (nblk_row * 8) + j * 8) = packed;
    s[r * nblk_row + j] = (uint8_t)code_s;
  }
}

int amax_grid(int64_t nblocks) {
  int64_t g = (nblocks + kThreads - 1) / kThreads;
  if (g > 1024) g = 1024;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

size_t quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return sizeof(uint32_t) * (size_t)amax_grid(rows * (cols / 16));
}

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* q, uint8_t* s, float* gscale, bool scale_given,
                           void* workspace, hipStream_t stream) {
  const int64_t nblk_row = cols / 16;
  const int64_t nblocks = rows * nblk_row;
  const int np = amax_grid(nblocks);
  if (!scale_given) {
    amax_kernel<<<np, kThreads, 0, stream>>>(x, dtype, rows, nblk_row, ld_x,
                                             reinterpret_cast<uint32_t*>(workspace));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int64_t eg = (nblocks + kThreads - 1) / kThreads;
  if (eg > 2048) eg = 2048;
  encode_kernel<<<(int)eg, kThreads, 0, stream>>>(
      x, dtype, rows, nblk_row, ld_x, q, s, gscale,
      reinterpret_cast<const uint32_t*>(workspace), np, scale_given ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4
