// Weight-streaming NVFP4 GEMM for few rows of x: the decode case (up to 64
// tokens per pass over the weights; the launcher runs up to two passes).
//
// The pages place these shapes far below the compute ridge: decode batches of
// 16-64 tokens reach a small fraction of the big-GEMM rate (magik.net "The
// Moment of Recalibration", "Input Knowledge", previous benchmark results).
// The kernel is therefore built to move the packed weights from HBM once, at
// full line width, and to hide the dequantise-and-multiply work under that
// stream:
//
//  * One workgroup owns 32 weight rows (an n-tile) over all of K.  Its 8 waves
//    split K in units of 256 elements; for the products, lane group q of a
//    wave holds the 64 contiguous elements [64q, 64q+64) of its row: 32
//    nibble bytes and 4 scale bytes.
//  * Every workgroup reads all of x, so at M = 32 a CU pulls as many
//    activation bytes (from L2) as weight bytes (from HBM).  Measured on the
//    MI355X, loads that cover half lines (4 lanes x 16 bytes of 16 rows)
//    make each activation byte cost about as much as a weight byte, while
//    loads of the same bytes by whole lines cost far less.  Activation
//    nibbles are therefore loaded by whole 128-byte lines (lane L: row L % 8
//    of the fragment's first or second eight rows, 16 bytes at 16 * (L / 8))
//    and moved into the product layout by two DPP row rotations per dword
//    pair; so are the weights' (their loads get faster by a little more than
//    the merges cost: M = 16 / 32 12.1 / 14.9 against 12.3 / 15.2 us).  Up
//    to 8 tokens both keep the direct layout (each lane loads its own 32
//    bytes, no merges): the activations are then few bytes, and whole-line
//    weights alone measured slower there (M = 1 11.4 against 11.1 us).
//  * Loads are software-pipelined one unit deep and ordered by first use
//    (activations, weight scales, then the first and the second 16 bytes of
//    each weight fragment), so a unit's products wait on the weight stream
//    piece by piece.  Deeper pipelines (more units in flight per wave) were
//    measured slower at every M.
//  * Products run on v_mfma_f32_16x16x32_f16 with weights as the 16-row A
//    operand and up to 64 tokens as one to four B operands; both sides are
//    dequantised exactly to fp16 in registers.  K is permuted identically on
//    both sides.
//  * The 8 per-wave partial tiles are summed through LDS in a fixed order, so
//    results are deterministic (no atomics, no split-K across workgroups).
#include "nvfp4_device.h"
#include "nvfp4_encode.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWG = 32;   // weight rows (output columns) per workgroup
constexpr int kUnitK = 256;      // K elements per wave step
// units per wave per round: 4 (K <= 8192 per round), 2 with four token
// fragments (their registers)
template <int NX>
constexpr int max_units() { return NX > 2 ? 2 : 4; }
constexpr uint32_t kOob = 0xFFFFFFF0u;  // offset past every operand (reads zero)
#ifndef NVFP4_DECODE_DEPTH
#define NVFP4_DECODE_DEPTH 1
#endif
constexpr int kDepth = NVFP4_DECODE_DEPTH;  // units in flight per wave

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

// One 256-element unit of one 16-row fragment, as held by a lane.
struct Unit {
  u32x4 q[2];  // 32 nibble bytes = 64 elements (MFMA steps 4i .. 4i+3 in q[i])
  uint32_t s;  // 4 scale bytes
};

// Byte offsets of one operand's 16-row fragment for this lane.
struct Frag {
  uint32_t q0, q1;  // the two 16-byte nibble loads of unit 0 (kOob past the rows)
  uint32_t s;       // the lane's 4 scale bytes of unit 0 (kOob past the rows)
};

// Fragment rows r0 .. r0+15 of an operand with `rows` rows.  Whole lines:
// nibble load h (0, 1) gives lane L the 16 bytes at 16 * (L / 8) of row
// r0 + 8h + L % 8 (merge_unit then sorts them).  Direct: lane (li, lq) =
// (L % 16, L / 16) loads bytes 32lq .. 32lq+31 of row r0 + li.  Either way
// the scale load gives lane (li, lq) bytes 4lq .. 4lq+3 of row r0 + li's
// unit scales.
template <bool kWhole>
__device__ __forceinline__ Frag make_frag(int r0, int rows, uint32_t qrow, uint32_t srow, int lane) {
  const int rs = r0 + (lane & 15);
  const uint32_t so = rs < rows ? (uint32_t)rs * srow + (uint32_t)(lane >> 4) * 4u : kOob;
  if constexpr (kWhole) {
    const int ra = r0 + (lane & 7), rb = ra + 8;
    const uint32_t col = (uint32_t)(lane >> 3) * 16u;
    return Frag{ra < rows ? (uint32_t)ra * qrow + col : kOob, rb < rows ? (uint32_t)rb * qrow + col : kOob, so};
  } else {
    // half lines: lane (li, lq) loads its own 32 bytes, no merge needed
    const uint32_t o = (uint32_t)rs * qrow + (uint32_t)(lane >> 4) * 32u;
    return Frag{rs < rows ? o : kOob, rs < rows ? o + 16u : kOob, so};
  }
}

// Loads a unit whose bytes sit uq (nibbles) and us (scales) past unit 0;
// offsets past the range read as zero.  Direct fragments: q[0], q[1] are the
// lane's own 32 bytes.  Whole-line fragments: the two loads are merged into
// the product layout later (merge_unit): lane l (row l % 16) needs chunks
// 2(l/16) and 2(l/16)+1 of its row, which lanes l and l ^ 8 hold between
// them (l % 16 < 8: a[l], a[l ^ 8]; else b[l ^ 8], b[l]).
__device__ __forceinline__ Unit load_unit(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                          const Frag& f, uint32_t uq, uint32_t us, bool in) {
  const u32x4 a = ld16(rq, in && f.q0 != kOob ? f.q0 + uq : kOob);
  const u32x4 b = ld16(rq, in && f.q1 != kOob ? f.q1 + uq : kOob);
  Unit r;
  r.s = ld4(rs, in && f.s != kOob ? f.s + us : kOob);
  r.q[0] = a;  // merged after the loads arrive (see merge_unit)
  r.q[1] = b;
  return r;
}

// DPP row rotation by 8 lanes (lane l of each 16-lane row reads lane l ^ 8),
// written only to the lanes of the bank mask; the others keep `old`.
constexpr int kRowRor8 = 0x128;
__device__ __forceinline__ void merge_unit(Unit& u) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int a = (int)u.q[0][d], b = (int)u.q[1][d];
    u.q[0][d] = (uint32_t)__builtin_amdgcn_update_dpp(a, b, kRowRor8, 0xF, 0xC, false);
    u.q[1][d] = (uint32_t)__builtin_amdgcn_update_dpp(b, a, kRowRor8, 0xF, 0x3, false);
  }
}

// The tokens (<= 16 * NX) against the 32-row tile, over all of K; leaves the
// wave's partial sums in acc[f][g] (weight fragment f, token fragment g).
// WL: both operands' fragments were made whole-line (make_frag<true>) and are
// merged after they land; otherwise both are direct (make_frag<false>).
template <int NX, bool WL>
__device__ __forceinline__ void chunk_partial(__amdgpu_buffer_rsrc_t wq, __amdgpu_buffer_rsrc_t ws,
                                              __amdgpu_buffer_rsrc_t xq, __amdgpu_buffer_rsrc_t xs,
                                              const Frag (&w)[2], const Frag (&x)[4], int nunits,
                                              int wave, f32x4 (&acc)[2][4]) {
  constexpr int kMaxUnits = max_units<NX>();
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = f32x4{0, 0, 0, 0};
  for (int ub = wave; ub < nunits; ub += kWaves * kMaxUnits) {
    Unit wu[kMaxUnits][2], xu[kMaxUnits][NX];
    auto load = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int u = ub + i * kWaves;
      const bool in = u < nunits;
      const uint32_t uq = (uint32_t)u * (kUnitK / 2), us = (uint32_t)u * (kUnitK / 16);
      // Order of a unit's loads = order of first use: the activations (from
      // L2), the weight scales, then the weight nibbles.  Whole-line weight
      // fragments go one after the other (fragment 0 is merged while 1
      // lands); direct ones give the first 16 bytes of both fragments (MFMA
      // steps 0-3) before the second (steps 4-7), so the products wait on the
      // weight stream piece by piece.
#pragma unroll
      for (int g = 0; g < NX; ++g) xu[i][g] = load_unit(xq, xs, x[g], uq, us, in);
#pragma unroll
      for (int f = 0; f < 2; ++f) wu[i][f].s = ld4(ws, in && w[f].s != kOob ? w[f].s + us : kOob);
      if constexpr (WL) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t o = h == 0 ? w[f].q0 : w[f].q1;
            wu[i][f].q[h] = ld16(wq, in && o != kOob ? o + uq : kOob);
          }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const uint32_t o = h == 0 ? w[f].q0 : w[f].q1;
            wu[i][f].q[h] = ld16(wq, in && o != kOob ? o + uq : kOob);
          }
      }
    };
    // Software pipeline, kDepth units in flight: the loads of unit
    // i + kDepth - 1 go out before the products of unit i.  Every unit is
    // multiplied, also those past K (their loads read zeros, which add exact
    // zeros), so there is no branch for the compiler to sink loads into, and
    // scheduling barriers keep each unit's loads at their place in the order.
    constexpr int kD = kDepth < kMaxUnits ? kDepth : kMaxUnits;
    static_for<kD>([&](auto ic) { load(ic); });
    static_for<kMaxUnits>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i > 0 && i + kD - 1 < kMaxUnits) load(std::integral_constant<int, i + kD - 1>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WL) {
#pragma unroll
        for (int g = 0; g < NX; ++g) merge_unit(xu[i][g]);
#pragma unroll
        for (int f = 0; f < 2; ++f) merge_unit(wu[i][f]);
      }
      Scales sw[2], sx[NX];
#pragma unroll
      for (int f = 0; f < 2; ++f) sw[f] = to_scales(wu[i][f].s);
#pragma unroll
      for (int g = 0; g < NX; ++g) sx[g] = to_scales(xu[i][g].s);
      // step T uses dword T % 4 of register T / 4; its scale is byte T / 2
      static_for<8>([&](auto tc) {
        constexpr int T = decltype(tc)::value, Q = T / 4, D = T % 4;
        const f16x8 a0 = dequant_step<T>(wu[i][0].q[Q][D], sw[0]);
        const f16x8 a1 = dequant_step<T>(wu[i][1].q[Q][D], sw[1]);
#pragma unroll
        for (int g = 0; g < NX; ++g) {
          const f16x8 b = dequant_step<T>(xu[i][g].q[Q][D], sx[g]);
          acc[0][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b, acc[0][g], 0, 0, 0);
          acc[1][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b, acc[1][g], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep each step's dequant beside its MFMAs
      });
    });
  }
}

__global__ __launch_bounds__(kThreads, 2) void gemm_decode_kernel(
    int N, int K, int M, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y, QuantOut qo) {
  __shared__ float red[kWaves][kRowsPerWG][32 + 1];
  __shared__ float yt[32][kRowsPerWG + 4];  // NVFP4 output: 32 tokens x 32 columns

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int n0 = (int)blockIdx.x * kRowsPerWG;

  const uint32_t qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
  const __amdgpu_buffer_rsrc_t wq = rsrc(b_q, (uint32_t)N * qrow), ws = rsrc(b_s, (uint32_t)N * srow);
  const __amdgpu_buffer_rsrc_t xq = rsrc(a_q, (uint32_t)M * qrow), xs = rsrc(a_s, (uint32_t)M * srow);
  const int nunits = K / kUnitK;
  const float alpha = a_g[0] * b_g[0];

  // weight rows of this lane's products: n0 + 16 f + li; token rows: 16 g + li.
  // More than 8 tokens: whole-line loads of both operands; up to 8 the
  // activations are few bytes and the direct layout needs no merges.
  Frag w[2], x[4];
  if (M > 8) {  // uniform
#pragma unroll
    for (int f = 0; f < 2; ++f) w[f] = make_frag<true>(n0 + 16 * f, N, qrow, srow, lane);
#pragma unroll
    for (int g = 0; g < 4; ++g) x[g] = make_frag<true>(16 * g, M, qrow, srow, lane);
  } else {
#pragma unroll
    for (int f = 0; f < 2; ++f) w[f] = make_frag<false>(n0 + 16 * f, N, qrow, srow, lane);
#pragma unroll
    for (int g = 0; g < 4; ++g) x[g] = make_frag<false>(16 * g, M, qrow, srow, lane);
  }

  f32x4 acc[2][4];
  if (M > 32) chunk_partial<4, true>(wq, ws, xq, xs, w, x, nunits, wave, acc);  // uniform
  else if (M > 16) chunk_partial<2, true>(wq, ws, xq, xs, w, x, nunits, wave, acc);
  else if (M > 8) chunk_partial<1, true>(wq, ws, xq, xs, w, x, nunits, wave, acc);
  else chunk_partial<1, false>(wq, ws, xq, xs, w, x, nunits, wave, acc);

  // Partial tiles -> LDS and a fixed-order sum over the waves, 32 tokens at
  // a time: acc[f][g] reg r is weight row 16f + 4*lq + r, token 16g + li.
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half * 32 >= M) break;  // uniform
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[wave][16 * f + 4 * lq + r][16 * g + li] = acc[f][2 * half + g][r];
    __syncthreads();
    // 1024 outputs (32 tokens x 32 weight rows), two per thread
#pragma unroll
    for (int h = 0; h < (32 * kRowsPerWG) / kThreads; ++h) {
      const int o = tid + h * kThreads;
      const int tok = 32 * half + (o >> 5), wr = o & 31;
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) s += red[v][wr][o >> 5];
      const int n = n0 + wr;
      if (y_dtype == 2) yt[o >> 5][wr] = s * alpha;
      else if (tok < M && n < N) store_out(y, (int64_t)tok * ld_y + n, s * alpha, y_dtype);
    }
    if (y_dtype == 2) {  // uniform
      // the same fp32 values, quantised: lane t of the first wave encodes
      // token t/2's block t%2 (16 columns) with the given global scale
      __syncthreads();
      if (tid < 64) {
        const int tok = 32 * half + (tid >> 1), c0 = n0 + 16 * (tid & 1);
        const float g = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(qo.g[0])));
        const enc::EncodeParams P = enc::make_params(g);
        const int mode = enc::encode_mode(g);
        enc::Block16 b;
#pragma unroll
        for (int e = 0; e < 16; ++e) b.v[e] = yt[tid >> 1][16 * (tid & 1) + e];
        if (tok < M && c0 < N) {
          uint8_t* qp = qo.q + (int64_t)tok * (N / 2) + c0 / 2;
          uint8_t* sp = qo.s + (int64_t)tok * (N / 16) + c0 / 16;
          if (mode == 1) enc::encode_block<1>(b, P, qp, sp);
          else if (mode == 0) enc::encode_block<0>(b, P, qp, sp);
          else enc::encode_block<2>(b, P, qp, sp);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gemm_decode(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                              void* y, int y_dtype, int64_t ld_y, hipStream_t stream, QuantOut qo) {
  const int64_t tiles = (N + kRowsPerWG - 1) / kRowsPerWG;
  // up to 64 tokens per launch; more rows go in 64-row passes over W (the
  // later passes find W in the Infinity Cache when it fits there)
  const size_t ysize = y_dtype == 0 ? 4 : 2;
  for (int64_t r0 = 0; r0 < M; r0 += 64) {
    const int64_t m = M - r0 < 64 ? M - r0 : 64;
    QuantOut qp = qo;
    if (y_dtype == 2) {
      qp.q += r0 * (N / 2);
      qp.s += r0 * (N / 16);
    }
    gemm_decode_kernel<<<(unsigned)tiles, kThreads, 0, stream>>>(
        (int)N, (int)K, (int)m, a.q + r0 * (K / 2), a.s + r0 * (K / 16), a.g, b.q, b.s, b.g,
        y_dtype == 2 ? y : static_cast<uint8_t*>(y) + r0 * ld_y * (int64_t)ysize, y_dtype, ld_y, qp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nvfp4
