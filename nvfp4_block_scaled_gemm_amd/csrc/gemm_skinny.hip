// Weight-streaming NVFP4 GEMM for few rows of x: the decode case (M <= 32)
// and the per-expert grouped case (mixture-of-experts, a handful of tokens
// per expert).
//
// The pages place these shapes far below the compute ridge: decode batches of
// 16-64 tokens reach a small fraction of the big-GEMM rate (magik.net "The
// Moment of Recalibration", "Input Knowledge", previous benchmark results),
// and a per-expert 32 x 2048 x 6144 GEMM is dozens of times under the ridge,
// so grouping the experts into one launch is the lever ("The Moment of
// Synthesis", "The Reasoning Process").  The kernel is therefore built to
// move the packed weights from HBM once, at full line width, with as many
// bytes in flight as possible:
//
//  * One workgroup owns 32 weight rows (an n-tile) of one group over all of
//    K.  Its 8 waves split K in units of 256 elements; per unit a lane loads
//    32 contiguous nibble bytes and 4 scale bytes of each of its two weight
//    rows, so four lanes cover a full 128-byte line of a row.  All of a
//    wave's units are loaded before the first is used.
//  * Products run on v_mfma_f32_16x16x32_f16 with weights as the 16-row A
//    operand and up to 32 tokens as one or two B operands; both sides are
//    dequantised exactly to fp16 in registers.  K is permuted identically on
//    both sides (lane group q of a unit holds elements [64q, 64q+64)).
//  * The 8 per-wave partial tiles are summed through LDS in a fixed order, so
//    results are deterministic (no atomics, no split-K across workgroups).
//  * Grouped: workgroup w takes group w / tiles_per_group; its rows are
//    [m_offsets[e], m_offsets[e+1]), processed 32 tokens at a time (weights
//    of later token chunks come back from cache, not HBM).
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWG = 32;   // weight rows (output columns) per workgroup
constexpr int kUnitK = 256;      // K elements per wave step
constexpr int kMaxUnits = 4;     // units held in registers per wave (K <= 8192 per round)

struct Unit {
  u32x4 q0, q1;  // 32 nibble bytes = 64 elements
  uint32_t s;    // 4 scale bytes
};

__device__ __forceinline__ Unit load_unit(const uint8_t* q_row, const uint8_t* s_row, int u,
                                          int lq, bool valid) {
  Unit r;
  if (valid) {
    const u32x4* p = reinterpret_cast<const u32x4*>(q_row + (int64_t)u * (kUnitK / 2) + lq * 32);
    r.q0 = p[0];
    r.q1 = p[1];
    r.s = *reinterpret_cast<const uint32_t*>(s_row + (int64_t)u * (kUnitK / 16) + lq * 4);
  } else {
    r.q0 = u32x4{0, 0, 0, 0};
    r.q1 = u32x4{0, 0, 0, 0};
    r.s = 0;
  }
  return r;
}

__device__ __forceinline__ uint32_t unit_word(const Unit& u, int t) {
  return t < 4 ? u.q0[t] : u.q1[t - 4];
}

// One 32-row x (<= 32 token) tile over all of K.
template <bool GROUPED>
__global__ __launch_bounds__(kThreads, 2) void gemm_skinny_kernel(
    int N, int K, int tiles_per_group, const int32_t* __restrict__ m_offsets, int64_t total_m,
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y) {
  __shared__ float red[kWaves][kRowsPerWG][32 + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int e = GROUPED ? (int)(blockIdx.x / tiles_per_group) : 0;
  const int nt = GROUPED ? (int)(blockIdx.x % tiles_per_group) : (int)blockIdx.x;
  const int n0 = nt * kRowsPerWG;

  int64_t row_begin = 0, row_end = total_m;
  if (GROUPED) {
    row_begin = m_offsets[e];
    row_end = m_offsets[e + 1];
    // rows outside [0, total_m) are never touched, whatever the offsets hold
    row_begin = row_begin < 0 ? 0 : (row_begin > total_m ? total_m : row_begin);
    row_end = row_end < row_begin ? row_begin : (row_end > total_m ? total_m : row_end);
  }
  if (row_end <= row_begin) return;  // empty group: the whole workgroup leaves

  const int64_t qstride = K / 2, sstride = K / 16;
  const uint8_t* bq = b_q + ((int64_t)e * N) * qstride;
  const uint8_t* bs = b_s + ((int64_t)e * N) * sstride;
  const int nunits = K / kUnitK;
  const float alpha = a_g[0] * b_g[e];

  // weight rows of this lane: n0 + 16*f + li, f = 0, 1
  const int wrow0 = n0 + li, wrow1 = n0 + 16 + li;
  const bool wv0 = wrow0 < N, wv1 = wrow1 < N;
  const uint8_t* wq0 = bq + (int64_t)wrow0 * qstride;
  const uint8_t* wq1 = bq + (int64_t)wrow1 * qstride;
  const uint8_t* ws0 = bs + (int64_t)wrow0 * sstride;
  const uint8_t* ws1 = bs + (int64_t)wrow1 * sstride;

  for (int64_t c0 = row_begin; c0 < row_end; c0 += 32) {
    const int ntok = (int)((row_end - c0) < 32 ? (row_end - c0) : 32);
    const bool two = ntok > 16;  // wave-uniform
    const int64_t xr0 = c0 + li, xr1 = c0 + 16 + li;
    const bool xv0 = li < ntok, xv1 = 16 + li < ntok;
    const uint8_t* xq0 = a_q + xr0 * qstride;
    const uint8_t* xq1 = a_q + xr1 * qstride;
    const uint8_t* xs0 = a_s + xr0 * sstride;
    const uint8_t* xs1 = a_s + xr1 * sstride;

    f32x4 acc00 = {0, 0, 0, 0}, acc01 = {0, 0, 0, 0}, acc10 = {0, 0, 0, 0},
          acc11 = {0, 0, 0, 0};

    for (int ub = wave; ub < nunits; ub += kWaves * kMaxUnits) {
      // issue every weight load of this round first
      Unit w0[kMaxUnits], w1[kMaxUnits];
#pragma unroll
      for (int i = 0; i < kMaxUnits; ++i) {
        const int u = ub + i * kWaves;
        const bool in = u < nunits;
        w0[i] = load_unit(wq0, ws0, u, lq, in && wv0);
        w1[i] = load_unit(wq1, ws1, u, lq, in && wv1);
      }
#pragma unroll
      for (int i = 0; i < kMaxUnits; ++i) {
        const int u = ub + i * kWaves;
        if (u >= nunits) break;
        const Unit x0 = load_unit(xq0, xs0, u, lq, xv0);
        Unit x1;
        if (two) x1 = load_unit(xq1, xs1, u, lq, xv1);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int sh = 8 * (t >> 1);
          const f16x8 fw0 = dequant8_scaled(unit_word(w0[i], t), scale_pair_bits((w0[i].s >> sh) & 0xFFu));
          const f16x8 fw1 = dequant8_scaled(unit_word(w1[i], t), scale_pair_bits((w1[i].s >> sh) & 0xFFu));
          const f16x8 fx0 = dequant8_scaled(unit_word(x0, t), scale_pair_bits((x0.s >> sh) & 0xFFu));
          acc00 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw0, fx0, acc00, 0, 0, 0);
          acc10 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw1, fx0, acc10, 0, 0, 0);
          if (two) {
            const f16x8 fx1 = dequant8_scaled(unit_word(x1, t), scale_pair_bits((x1.s >> sh) & 0xFFu));
            acc01 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw0, fx1, acc01, 0, 0, 0);
            acc11 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw1, fx1, acc11, 0, 0, 0);
          }
        }
      }
    }

    // partial tiles -> LDS: acc[f][g] reg r is weight row 16f + 4*lq + r, token 16g + li
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      red[wave][4 * lq + r][li] = acc00[r];
      red[wave][16 + 4 * lq + r][li] = acc10[r];
      red[wave][4 * lq + r][16 + li] = acc01[r];
      red[wave][16 + 4 * lq + r][16 + li] = acc11[r];
    }
    __syncthreads();
    // 1024 outputs (32 tokens x 32 weight rows), two per thread, summed over
    // the waves in a fixed order
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = tid + h * kThreads;
      const int tok = o >> 5, wr = o & 31;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += red[w][wr][tok];
      const int n = n0 + wr;
      if (tok < ntok && n < N) store_out(y, (c0 + tok) * ld_y + n, s * alpha, y_dtype);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gemm_decode(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                              void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
  const int64_t tiles = (N + kRowsPerWG - 1) / kRowsPerWG;
  gemm_skinny_kernel<false><<<(unsigned)tiles, kThreads, 0, stream>>>(
      (int)N, (int)K, (int)tiles, nullptr, M, a.q, a.s, a.g, b.q, b.s, b.g, y, y_dtype, ld_y);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(int32_t G, const int32_t* m_offsets, int64_t total_m, int64_t N,
                               int64_t K, PackedOperand a, PackedOperand b, void* y, int y_dtype,
                               int64_t ld_y, hipStream_t stream) {
  const int64_t tiles = (N + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t grid = tiles * G;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  gemm_skinny_kernel<true><<<(unsigned)grid, kThreads, 0, stream>>>(
      (int)N, (int)K, (int)tiles, m_offsets, total_m, a.q, a.s, a.g, b.q, b.s, b.g, y, y_dtype,
      ld_y);
  return hipGetLastError();
}

}  // namespace nvfp4
