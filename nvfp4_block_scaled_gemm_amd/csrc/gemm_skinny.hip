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
//    K.  Its 8 waves split K in units of 256 elements; per unit a lane holds
//    32 contiguous nibble bytes and 4 scale bytes of each of its two weight
//    rows, so four lanes cover a full 128-byte line of a row.  Every weight
//    and activation load of a wave (up to 4 units each) is issued before the
//    first is used, so a CU has its whole weight slice in flight at once.
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
constexpr int kMaxUnits = 4;     // units per wave per round (K <= 8192 per round)

struct Unit {
  u32x4 q0, q1;  // 32 nibble bytes = 64 elements (MFMA steps 0-3, 4-7)
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

template <int T>
__device__ __forceinline__ uint32_t unit_word(const Unit& u) {
  if constexpr (T < 4) return u.q0[T];
  else return u.q1[T - 4];
}

struct Rows {
  const uint8_t *q0, *q1, *s0, *s1;  // two rows (fragments 0 and 1) of one operand
  bool v0, v1;
};

// One token chunk (<= 16 * NX tokens) of the 32-row tile, over all of K;
// leaves the wave's partial sums in acc[f][g] (weight fragment f, token
// fragment g).
template <int NX>
__device__ __forceinline__ void chunk_partial(const Rows& w, const Rows& x, int nunits, int wave,
                                              int lq, f32x4 (&acc)[2][2]) {
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[f][g] = f32x4{0, 0, 0, 0};
  for (int ub = wave; ub < nunits; ub += kWaves * kMaxUnits) {
    Unit w0[kMaxUnits], w1[kMaxUnits], x0[kMaxUnits], x1[kMaxUnits];
    // every load of the round first, unit by unit (weights, then that
    // unit's activations), so unit i's products wait only for loads issued
    // up to unit i and overlap the later units' transfers
#pragma unroll
    for (int i = 0; i < kMaxUnits; ++i) {
      const int u = ub + i * kWaves;
      const bool in = u < nunits;
      w0[i] = load_unit(w.q0, w.s0, u, lq, in && w.v0);
      w1[i] = load_unit(w.q1, w.s1, u, lq, in && w.v1);
      x0[i] = load_unit(x.q0, x.s0, u, lq, in && x.v0);
      if constexpr (NX == 2) x1[i] = load_unit(x.q1, x.s1, u, lq, in && x.v1);
    }
#pragma unroll
    for (int i = 0; i < kMaxUnits; ++i) {
      if (ub + i * kWaves >= nunits) break;
      const Scales sw0 = to_scales(w0[i].s), sw1 = to_scales(w1[i].s), sx0 = to_scales(x0[i].s);
      Scales sx1;
      if constexpr (NX == 2) sx1 = to_scales(x1[i].s);
      static_for<8>([&](auto tc) {
        constexpr int T = decltype(tc)::value;
        const f16x8 a0 = dequant_step<T>(unit_word<T>(w0[i]), sw0);
        const f16x8 a1 = dequant_step<T>(unit_word<T>(w1[i]), sw1);
        const f16x8 b0 = dequant_step<T>(unit_word<T>(x0[i]), sx0);
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, acc[0][0], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b0, acc[1][0], 0, 0, 0);
        if constexpr (NX == 2) {
          const f16x8 b1 = dequant_step<T>(unit_word<T>(x1[i]), sx1);
          acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b1, acc[0][1], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[1][1], 0, 0, 0);
        }
      });
    }
  }
}

template <bool GROUPED>
__global__ __launch_bounds__(kThreads, 2) void gemm_skinny_kernel(
    int N, int K, int tiles_per_group, const int32_t* __restrict__ m_offsets, int64_t total_m,
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y) {
  __shared__ float red[kWaves][kRowsPerWG][32 + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  Rows w;
  {
    const int r0 = n0 + li, r1 = n0 + 16 + li;
    w.v0 = r0 < N;
    w.v1 = r1 < N;
    w.q0 = bq + (int64_t)r0 * qstride;
    w.q1 = bq + (int64_t)r1 * qstride;
    w.s0 = bs + (int64_t)r0 * sstride;
    w.s1 = bs + (int64_t)r1 * sstride;
  }

  for (int64_t c0 = row_begin; c0 < row_end; c0 += 32) {
    const int ntok = (int)((row_end - c0) < 32 ? (row_end - c0) : 32);
    Rows x;
    x.v0 = li < ntok;
    x.v1 = 16 + li < ntok;
    x.q0 = a_q + (c0 + li) * qstride;
    x.q1 = a_q + (c0 + 16 + li) * qstride;
    x.s0 = a_s + (c0 + li) * sstride;
    x.s1 = a_s + (c0 + 16 + li) * sstride;

    f32x4 acc[2][2];
    if (ntok > 16) chunk_partial<2>(w, x, nunits, wave, lq, acc);  // wave-uniform
    else chunk_partial<1>(w, x, nunits, wave, lq, acc);

    // partial tiles -> LDS: acc[f][g] reg r is weight row 16f + 4*lq + r,
    // token 16g + li
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][16 * f + 4 * lq + r][16 * g + li] = acc[f][g][r];
    __syncthreads();
    // 1024 outputs (32 tokens x 32 weight rows), two per thread, summed over
    // the waves in a fixed order
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = tid + h * kThreads;
      const int tok = o >> 5, wr = o & 31;
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) s += red[v][wr][tok];
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

}  // namespace nvfp4
