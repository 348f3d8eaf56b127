// MXFP4 variant: 32-element blocks with power-of-two (E8M0) scales, the
// block shape gfx950's scaled FP4 matrix instructions consume natively.
// The pages define NVFP4 only (FP4 packs twice FP8's values: magik.net "The
// 3.7 PFLOPS Revelation", "Input Knowledge", item 2); this variant follows
// the microscaling definition instead of NVFP4's E4M3 scales:
//   E      = floor(log2(amax_b)) - 2, clamped to [-127, 127] (-127 for a
//            zero block); scale byte E + 127
//   code_i = E2M1 rounding (nearest, ties to the even code, saturating at
//            6, sign kept) of x_i / 2^E
//   a block holding a NaN or an infinity: scale byte 255, nibbles 0
// y[m, n] = sum_k A(m, k) B(n, k), no per-tensor scale.
//
// The quantiser needs no tensor-wide pass (the scale depends on its block
// only), so it is a single streaming kernel: one thread per block of 32,
// whose division by 2^E is exact, so the hardware E2M1 encoder's round-to-
// nearest-even on the scaled value is the exact rounding.  The general GEMM
// below serves shapes the matrix-core kernel (gemm_mfma.hip) does not take.
#include "nvfp4_device.h"
#include "nvfp4_encode.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

// floor(log2(a)) of a positive finite fp32 given by its bits (subnormals
// included), exactly.
__device__ __forceinline__ int floor_log2_bits(uint32_t bits) {
  const int ef = (int)(bits >> 23);
  return ef != 0 ? ef - 127 : (31 - __builtin_clz(bits)) - 149;
}

// Eight values -> one dword of nibbles (element 2p in the low nibble of
// byte p), each multiplied by `inv` (a power of two, so exactly).
__device__ __forceinline__ uint32_t encode8(const float* v, float inv) {
  uint32_t w = 0;
  static_for<4>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2 * p] * inv, v[2 * p + 1] * inv, 1.0f, p);
  });
  return w;
}

__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(
    const void* __restrict__ x, int dtype, int64_t rows, int64_t nblk_row, int64_t ld_x,
    uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t total = rows * nblk_row;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * kThreads) {
    const int64_t r = c / nblk_row, j = c - r * nblk_row;
    enc::Block16 lo, hi;
    enc::load_block(x, dtype, r * ld_x + j * 32, lo);
    enc::load_block(x, dtype, r * ld_x + j * 32 + 16, hi);
    // |x| bits order like the values; NaN and infinity sit at 0x7F800000
    // and above
    const uint32_t m = max(enc::block_amax_bits(lo), enc::block_amax_bits(hi));
    u32x4 out = {0, 0, 0, 0};
    uint32_t sb = 255;
    if (m < 0x7F800000u) {
      int E = m == 0 ? -127 : floor_log2_bits(m) - 2;
      E = E < -127 ? -127 : (E > 127 ? 127 : E);
      sb = (uint32_t)(E + 127);
      // 2^-E is a normal fp32 for E in [-127, 125] (the largest finite
      // fp32 block gives E = 125); values scaled below fp32's normal range
      // are far below E2M1's first midpoint (0.25) either way
      const float inv = __uint_as_float((uint32_t)(127 - E) << 23);
      out[0] = encode8(lo.v, inv);
      out[1] = encode8(lo.v + 8, inv);
      out[2] = encode8(hi.v, inv);
      out[3] = encode8(hi.v + 8, inv);
    }
    *reinterpret_cast<u32x4*>(q + r * (nblk_row * 16) + j * 16) = out;
    s[r * nblk_row + j] = (uint8_t)sb;
  }
}

// One output per thread: per block, the integer sum of products of 2x E2M1
// magnitudes (exact), times 2^(sa + sb - 254) / 4, accumulated in fp32 in
// block order.  A NaN scale byte makes the output NaN.
__global__ __launch_bounds__(kThreads) void mx_gemm_generic_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_q,
    const uint8_t* __restrict__ a_s, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, void* __restrict__ y, int y_dtype, int64_t ld_y,
    int64_t m_base) {
  const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  const int64_t m = m_base + (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  if (m >= M || n >= N) return;
  const int64_t nblk = K / 32;
  const uint8_t* aq = a_q + m * (K / 2);
  const uint8_t* bq = b_q + n * (K / 2);
  float acc = 0.0f;
  for (int64_t blk = 0; blk < nblk; ++blk) {
    int isum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t xa = aq[blk * 16 + j], xb = bq[blk * 16 + j];
      isum += e2m1_x2(xa & 15u) * e2m1_x2(xb & 15u);
      isum += e2m1_x2(xa >> 4) * e2m1_x2(xb >> 4);
    }
    const int sa = a_s[m * nblk + blk], sb = b_s[n * nblk + blk];
    acc += (sa == 255 || sb == 255) ? __builtin_nanf("")
                                    : __builtin_ldexpf((float)isum * 0.25f, sa + sb - 254);
  }
  store_out(y, m * ld_y + n, acc, y_dtype);
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t* q, uint8_t* s, hipStream_t stream) {
  const int64_t nblk_row = cols / 32;
  const int64_t total = rows * nblk_row;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + kThreads - 1) / kThreads;
  if (grid > 65536) grid = 65536;  // grid-stride beyond
  mx_quantize_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(x, dtype, rows, nblk_row, ld_x, q,
                                                              s);
  return hipGetLastError();
}

hipError_t launch_mx_gemm_generic(int64_t M, int64_t N, int64_t K, const uint8_t* a_q,
                                  const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                                  void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
  const int64_t max_rows = 65535LL * 16;  // grid.y limit: larger M in row chunks
  for (int64_t m0 = 0; m0 < M; m0 += max_rows) {
    const int64_t rows = (M - m0 < max_rows) ? (M - m0) : max_rows;
    dim3 grid((unsigned)((N + 15) / 16), (unsigned)((rows + 15) / 16));
    mx_gemm_generic_kernel<<<grid, kThreads, 0, stream>>>(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype,
                                                           ld_y, m0);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace nvfp4
