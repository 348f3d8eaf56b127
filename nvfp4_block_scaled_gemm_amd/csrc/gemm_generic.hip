// General NVFP4 GEMM for shapes the tiled kernels do not take (K not a
// multiple of the tile depth, unaligned rows).  One thread per output element;
// each 16-element block product is formed exactly in integers and scaled
// exactly in fp32, and the block contributions are summed in fp32 in K order.
//
// y[m, n] = fl32(ga * gb) * sum_k A(m, k) B(n, k)   (kernelindex "NVFP4 linear
// layer", description: y = x @ W^T with E2M1 operands and E4M3FN scales per
// 16 elements).  With m_offsets given, row m uses weight group e where
// m_offsets[e] <= m < m_offsets[e+1] (grouped form), and with row_index
// given it reads activation row row_index[m] (a zero row if that index is
// outside [0, a_rows)).  With NVFP4 output (dense form only) the same fp32
// values are quantised in 16-column blocks by the quantiser's encoder.
#include "nvfp4_device.h"
#include "nvfp4_encode.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

// One output y[m, n] (fp32, scaled).
__device__ __forceinline__ float dot(int64_t M, int64_t N, int64_t K,
                                     const uint8_t* __restrict__ a_q,
                                     const uint8_t* __restrict__ a_s,
                                     const uint8_t* __restrict__ b_q,
                                     const uint8_t* __restrict__ b_s,
                                     const int32_t* __restrict__ m_offsets, int32_t G,
                                     const int32_t* __restrict__ row_index, int64_t a_rows,
                                     int64_t m, int64_t n, const float* __restrict__ a_g,
                                     const float* __restrict__ b_g) {
  int64_t e = 0;
  if (m_offsets != nullptr) {
    // last group e with m_offsets[e] <= m (non-decreasing offsets)
    int32_t lo = 0, hi = G - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if ((int64_t)m_offsets[mid] <= m) lo = mid; else hi = mid - 1;
    }
    e = lo;
  }
  const int64_t nblk = K / 16;
  int64_t src = m;
  bool a_ok = true;
  if (row_index != nullptr) {
    src = row_index[m];
    a_ok = src >= 0 && src < a_rows;
    if (!a_ok) src = 0;
  }
  const uint8_t* aq = a_q + src * (K / 2);
  const uint8_t* as = a_s + src * nblk;
  const uint8_t* bq = b_q + (e * N + n) * (K / 2);
  const uint8_t* bs = b_s + (e * N + n) * nblk;
  float acc = 0.0f;
  for (int64_t blk = 0; a_ok && blk < nblk; ++blk) {
    int isum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t xa = aq[blk * 8 + j], xb = bq[blk * 8 + j];
      isum += e2m1_x2(xa & 15u) * e2m1_x2(xb & 15u);
      isum += e2m1_x2(xa >> 4) * e2m1_x2(xb >> 4);
    }
    const float sc = e4m3_to_f32(as[blk]) * e4m3_to_f32(bs[blk]);  // exact
    acc += sc * ((float)isum * 0.25f);                                 // exact term
  }
  const float alpha = a_g[0] * b_g[e];
  return acc * alpha;
}

__global__ __launch_bounds__(256) void gemm_generic_kernel(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ a_q,
    const uint8_t* __restrict__ a_s, const float* __restrict__ a_g,
    const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s,
    const float* __restrict__ b_g, const int32_t* __restrict__ m_offsets, int32_t G,
    const int32_t* __restrict__ row_index, int64_t a_rows, void* __restrict__ y, int y_dtype,
    int64_t ld_y, QuantOut qo, int64_t m_base) {
  // rows m_base + blockIdx.y * 16 + ... of the whole problem (grid.y is
  // limited, so large M is launched in row chunks)
  const int64_t n = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  const int64_t m = m_base + (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  const bool in = m < M && n < N;
  if (!in && y_dtype != 2) return;  // the NVFP4 writer needs every thread at its barrier
  const float v = in ? dot(M, N, K, a_q, a_s, b_q, b_s, m_offsets, G, row_index, a_rows, m, n,
                           a_g, b_g)
                     : 0.0f;
  if (y_dtype != 2) {
    store_out(y, m * ld_y + n, v, y_dtype);
    return;
  }
  // NVFP4 output: the workgroup's 16 x 16 values go through LDS; thread t < 16
  // encodes row t's 16-column block with the given global scale
  __shared__ float tile[16][17];
  tile[threadIdx.x >> 4][threadIdx.x & 15] = v;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int64_t row = m_base + (int64_t)blockIdx.y * 16 + threadIdx.x, c0 = (int64_t)blockIdx.x * 16;
    const float g = qo.g[0];
    const enc::EncodeParams P = enc::make_params(g);
    const int mode = enc::encode_mode(g);
    enc::Block16 b;
#pragma unroll
    for (int e = 0; e < 16; ++e) b.v[e] = tile[threadIdx.x][e];
    if (row < M && c0 < N) {
      uint8_t* qp = qo.q + row * (N / 2) + c0 / 2;
      uint8_t* sp = qo.s + row * (N / 16) + c0 / 16;
      if (mode == 1) enc::encode_block<1>(b, P, qp, sp);
      else if (mode == 0) enc::encode_block<0>(b, P, qp, sp);
      else enc::encode_block<2>(b, P, qp, sp);
    }
  }
}

hipError_t launch(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                  const int32_t* m_offsets, int32_t G, const int32_t* row_index, int64_t a_rows,
                  void* y, int y_dtype, int64_t ld_y, hipStream_t stream, QuantOut qo) {
  // grid.y is limited to 65535 row tiles; larger M is launched in row
  // chunks, each told its first row (pointers stay those of the whole
  // problem, so the group search and the row index see global rows)
  const int64_t max_rows = 65535LL * 16;
  for (int64_t m0 = 0; m0 < M; m0 += max_rows) {
    const int64_t rows = (M - m0 < max_rows) ? (M - m0) : max_rows;
    dim3 grid((unsigned)((N + 15) / 16), (unsigned)((rows + 15) / 16));
    gemm_generic_kernel<<<grid, 256, 0, stream>>>(M, N, K, a.q, a.s, a.g, b.q, b.s, b.g,
                                                   m_offsets, G, row_index, a_rows, y, y_dtype,
                                                   ld_y, qo, m0);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_generic(int64_t M, int64_t N, int64_t K, PackedOperand a,
                               PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                               hipStream_t stream, QuantOut qo) {
  return launch(M, N, K, a, b, nullptr, 1, nullptr, M, y, y_dtype, ld_y, stream, qo);
}

hipError_t launch_gemm_grouped_generic(int32_t G, const int32_t* m_offsets,
                                       const int32_t* row_index, int64_t total_m, int64_t a_rows,
                                       int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                                       void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
  return launch(total_m, N, K, a, b, m_offsets, G, row_index,
                row_index != nullptr ? a_rows : total_m, y, y_dtype, ld_y, stream, QuantOut{});
}

}  // namespace nvfp4
