// Grouped (per-expert) NVFP4 GEMM for mixture-of-experts layers.
//
// Each expert sees only a handful of tokens (magik.net "The Moment of
// Recalibration", "Input Knowledge": 256 experts, 8 per token, ~16 tokens per
// expert at 512 concurrent requests), so every per-expert GEMM sits far
// below the compute ridge and the only lever is to run them all as one
// grouped launch ("The Moment of Synthesis", "The Reasoning Process").  The
// job is then a pure weight stream: 3.6 GB of packed gate_up weights per
// layer must move from HBM at full rate, with the small dequantise-and-MFMA
// work hidden under it.
//
// Design (persistent, barrier-free):
//  * Work items are (expert e, 32-row weight tile); a wave owns an item over
//    all of K and all of the expert's tokens, so no partial sums ever cross
//    waves.  The waves of the grid walk the item list with a fixed stride;
//    experts without tokens are skipped.
//  * A wave's jobs are (item, 32-token chunk, 256-element K unit).  Each job
//    brings 4.5 KB of packed weights into a private 3-slot LDS ring with
//    buffer-to-LDS loads (4 x 16 B + 2 x 4 B per lane) and the chunk's
//    activation fragments into registers with buffer loads; out-of-range rows
//    read as zero.  Loads run two jobs ahead and every job issues the same 12
//    memory instructions (finished items pad with out-of-range loads), so one
//    fixed s_waitcnt per job suffices.
//  * A job dequantises both operands exactly to fp16 in registers and issues
//    v_mfma_f32_16x16x32_f16: two 16-row weight fragments x one or two
//    16-token fragments, 8 steps per unit.  K is permuted identically on both
//    sides (lane group q of a unit holds elements [64q, 64q+64)).
//  * After the last unit of an item-chunk the wave scales by ga * gb[e] and
//    stores its 32 x ntok outputs.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;                        // weight rows per item
constexpr int kUnitK = 256;                      // K elements per job
constexpr int kSlots = 3;                        // LDS ring depth per wave
constexpr int kSlotNib = kRows * (kUnitK / 2);   // 4096 B of nibbles
constexpr int kSlotBytes = kSlotNib + kRows * (kUnitK / 16);  // + 512 B of scales
constexpr int kWaveLds = kSlots * kSlotBytes;
constexpr int kLoadsPerJob = 12;                 // memory instructions per job
constexpr uint32_t kOob = 0xFFFFFFF0u;           // offset past every operand

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16(const void* p, uint32_t bytes, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(p, bytes), (lds_void_ptr)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(const void* p, uint32_t bytes, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(p, bytes), (lds_void_ptr)lds, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ u32x4 ld16(const void* p, uint32_t bytes, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(p, bytes), voff, 0, 0));
}
__device__ __forceinline__ uint32_t ld4(const void* p, uint32_t bytes, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc(p, bytes), voff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A wave's position in its job sequence (all fields wave-uniform).
struct Cursor {
  int item;              // global item id (>= n_items: finished)
  int e, n0;             // expert and first weight row of the item
  int r0, r1;            // the expert's token rows [r0, r1)
  int c0;                // first token row of the current chunk
  int u;                 // current K unit
};

struct Shape {
  int N, nunits, tiles, n_items, stride;
  int64_t total_m;
};

// Expert rows of item `it`, clamped into [0, total_m) whatever the offsets
// hold.  The expert index is made explicitly scalar so the two offsets come
// in through the scalar cache (their wait never drains the vector loads).
__device__ __forceinline__ void item_rows(const Shape& sh, const int32_t* __restrict__ m_offsets,
                                          int it, Cursor& c) {
  c.item = it;
  c.e = __builtin_amdgcn_readfirstlane(it / sh.tiles);
  c.n0 = (it - c.e * sh.tiles) * kRows;
  int64_t a = m_offsets[c.e], b = m_offsets[c.e + 1];
  a = a < 0 ? 0 : (a > sh.total_m ? sh.total_m : a);
  b = b < a ? a : (b > sh.total_m ? sh.total_m : b);
  c.r0 = (int)a;
  c.r1 = (int)b;
}

// First item at or after `it` (stepping by the grid stride) with tokens.
__device__ __forceinline__ void seek_item(const Shape& sh, const int32_t* __restrict__ m_offsets,
                                          int it, Cursor& c) {
  for (; it < sh.n_items; it += sh.stride) {
    item_rows(sh, m_offsets, it, c);
    if (c.r1 > c.r0) {
      c.c0 = c.r0;
      c.u = 0;
      return;
    }
  }
  c.item = sh.n_items;
}

__device__ __forceinline__ void advance(const Shape& sh, const int32_t* __restrict__ m_offsets,
                                        Cursor& c) {
  if (c.item >= sh.n_items) return;
  if (++c.u < sh.nunits) return;
  c.u = 0;
  c.c0 += 32;
  if (c.c0 < c.r1) return;
  seek_item(sh, m_offsets, c.item + sh.stride, c);
}

struct XFrags {
  u32x4 q0[2], q1[2];  // token fragments 0, 1: 32 nibble bytes each
  uint32_t s[2];       // their 4 scale bytes
};

__global__ __launch_bounds__(kThreads, 2) void gemm_grouped_kernel(
    Shape sh, const int32_t* __restrict__ m_offsets, int K, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lq = lane >> 4;
  uint8_t* ring = smem + wave * kWaveLds;

  const uint32_t qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
  const uint32_t wq_bytes = (uint32_t)sh.N * qrow, ws_bytes = (uint32_t)sh.N * srow;
  const uint32_t xq_bytes = (uint32_t)sh.total_m * qrow, xs_bytes = (uint32_t)sh.total_m * srow;
  const float ga = a_g[0];

  // per-lane parts of the weight load offsets (row within the item, byte
  // within the unit); direct load k of 16 B covers rows 8k .. 8k+7
  const uint32_t wrow16 = (uint32_t)(lane >> 3), wchunk = (uint32_t)(lane & 7) * 16;
  const uint32_t wrow4 = (uint32_t)(lane >> 2), wpart = (uint32_t)(lane & 3) * 4;

  XFrags xs[kSlots];

  // Loads of the job at `c` into slot S: weights to LDS, activations to
  // registers.  Always kLoadsPerJob memory instructions.
  auto issue = [&](const Cursor& c, auto sc) {
    constexpr int S = decltype(sc)::value;
    const bool live = c.item < sh.n_items;
    const int e = live ? c.e : 0;
    const uint8_t* wq = b_q + (int64_t)e * sh.N * qrow;
    const uint8_t* ws = b_s + (int64_t)e * sh.N * srow;
    uint8_t* slot = ring + S * kSlotBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t row = (uint32_t)(c.n0) + 8u * k + wrow16;
      dma16(wq, wq_bytes, live ? row * qrow + (uint32_t)c.u * 128u + wchunk : kOob,
            slot + k * 1024);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t row = (uint32_t)(c.n0) + 16u * k + wrow4;
      dma4(ws, ws_bytes, live ? row * srow + (uint32_t)c.u * 16u + wpart : kOob,
           slot + kSlotNib + k * 256);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int t = c.c0 + 16 * g + li;
      const bool ok = live && t < c.r1;
      const uint32_t qo = ok ? (uint32_t)t * qrow + (uint32_t)c.u * 128u + (uint32_t)lq * 32u : kOob;
      const uint32_t so = ok ? (uint32_t)t * srow + (uint32_t)c.u * 16u + (uint32_t)lq * 4u : kOob;
      xs[S].q0[g] = ld16(a_q, xq_bytes, qo);
      xs[S].q1[g] = ld16(a_q, xq_bytes, ok ? qo + 16u : kOob);
      xs[S].s[g] = ld4(a_s, xs_bytes, so);
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[f][g] = f32x4{0, 0, 0, 0};

  // One job from slot S (its loads have landed), then the item-chunk
  // epilogue if this was its last unit.
  auto compute = [&](const Cursor& c, auto sc) {
    constexpr int S = decltype(sc)::value;
    const uint8_t* slot = ring + S * kSlotBytes;
    u32x4 wlo[2], whi[2];
    Scales sw[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int row = 16 * f + li;
      wlo[f] = *reinterpret_cast<const u32x4*>(slot + row * 128 + lq * 32);
      whi[f] = *reinterpret_cast<const u32x4*>(slot + row * 128 + lq * 32 + 16);
      sw[f] = to_scales(*reinterpret_cast<const uint32_t*>(slot + kSlotNib + row * 16 + lq * 4));
    }
    const Scales sx0 = to_scales(xs[S].s[0]);
    const int ntok = min(32, c.r1 - c.c0);
    if (ntok > 16) {  // wave-uniform
      const Scales sx1 = to_scales(xs[S].s[1]);
      static_for<8>([&](auto tc) {
        constexpr int T = decltype(tc)::value;
        const uint32_t w0 = T < 4 ? wlo[0][T & 3] : whi[0][T & 3];
        const uint32_t w1 = T < 4 ? wlo[1][T & 3] : whi[1][T & 3];
        const uint32_t x0 = T < 4 ? xs[S].q0[0][T & 3] : xs[S].q1[0][T & 3];
        const uint32_t x1 = T < 4 ? xs[S].q0[1][T & 3] : xs[S].q1[1][T & 3];
        const f16x8 a0 = dequant_step<T>(w0, sw[0]), a1 = dequant_step<T>(w1, sw[1]);
        const f16x8 b0 = dequant_step<T>(x0, sx0), b1 = dequant_step<T>(x1, sx1);
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, acc[0][0], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b0, acc[1][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[1][1], 0, 0, 0);
      });
    } else {
      static_for<8>([&](auto tc) {
        constexpr int T = decltype(tc)::value;
        const uint32_t w0 = T < 4 ? wlo[0][T & 3] : whi[0][T & 3];
        const uint32_t w1 = T < 4 ? wlo[1][T & 3] : whi[1][T & 3];
        const uint32_t x0 = T < 4 ? xs[S].q0[0][T & 3] : xs[S].q1[0][T & 3];
        const f16x8 a0 = dequant_step<T>(w0, sw[0]), a1 = dequant_step<T>(w1, sw[1]);
        const f16x8 b0 = dequant_step<T>(x0, sx0);
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, acc[0][0], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b0, acc[1][0], 0, 0, 0);
      });
    }
    if (c.u == sh.nunits - 1) {
      // acc[f][g] reg r: weight row n0 + 16f + 4*lq + r, token c0 + 16g + li
      const float alpha = ga * b_g[c.e];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int tok = 16 * g + li;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = c.n0 + 16 * f + 4 * lq + r;
            if (tok < ntok && n < sh.N)
              store_out(y, (int64_t)(c.c0 + tok) * ld_y + n, acc[f][g][r] * alpha, y_dtype);
          }
          acc[f][g] = f32x4{0, 0, 0, 0};
        }
    }
  };

  Shape shl = sh;
  Cursor lc, cc;
  seek_item(shl, m_offsets, blockIdx.x * kWaves + wave, lc);
  cc = lc;
  issue(lc, std::integral_constant<int, 0>{});
  advance(shl, m_offsets, lc);
  issue(lc, std::integral_constant<int, 1>{});
  advance(shl, m_offsets, lc);
  // jobs rotate through slots 0, 1, 2; the loads of job j+2 go out before
  // job j waits for its own (two younger jobs may stay in flight)
  while (cc.item < shl.n_items) {
    issue(lc, std::integral_constant<int, 2>{});
    advance(shl, m_offsets, lc);
    wait_vmcnt<2 * kLoadsPerJob>();
    compute(cc, std::integral_constant<int, 0>{});
    advance(shl, m_offsets, cc);
    if (cc.item >= shl.n_items) break;
    issue(lc, std::integral_constant<int, 0>{});
    advance(shl, m_offsets, lc);
    wait_vmcnt<2 * kLoadsPerJob>();
    compute(cc, std::integral_constant<int, 1>{});
    advance(shl, m_offsets, cc);
    if (cc.item >= shl.n_items) break;
    issue(lc, std::integral_constant<int, 1>{});
    advance(shl, m_offsets, lc);
    wait_vmcnt<2 * kLoadsPerJob>();
    compute(cc, std::integral_constant<int, 2>{});
    advance(shl, m_offsets, cc);
  }
  wait_vmcnt<0>();  // padding loads land before the wave exits
}

}  // namespace

hipError_t launch_gemm_grouped(int32_t G, const int32_t* m_offsets, int64_t total_m, int64_t N,
                               int64_t K, PackedOperand a, PackedOperand b, void* y, int y_dtype,
                               int64_t ld_y, hipStream_t stream) {
  static int num_cu = 0;  // compute units of the current device (one query per process)
  if (num_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    num_cu = n;
  }
  const int64_t tiles = (N + kRows - 1) / kRows;
  const int64_t n_items = tiles * G;
  if (n_items > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int smem = kWaves * kWaveLds;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)gemm_grouped_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  int64_t grid = ((n_items + kWaves - 1) / kWaves);
  if (grid > num_cu) grid = num_cu;  // persistent: one workgroup per CU
  Shape sh{(int)N, (int)(K / kUnitK), (int)tiles, (int)n_items, (int)grid * kWaves, total_m};
  gemm_grouped_kernel<<<(unsigned)grid, kThreads, smem, stream>>>(sh, m_offsets, (int)K, a.q, a.s, a.g, b.q,
                                                                  b.s, b.g, y, y_dtype, ld_y);
  return hipGetLastError();
}

}  // namespace nvfp4
