// NVFP4 GEMM for large M on the gfx950 matrix cores.
//
// y[m, n] = fl32(ga * gb) * sum_k A(m, k) B(n, k), A = x [M, K], B = W [N, K]
// (kernelindex "NVFP4 linear layer", description).  The pages' kernels
// (CUTLASS / Colfax on SM120, magik.net "The Moment of Synthesis", "The
// Context That Led Here") consume FP4 natively with 128x128 tiles bounded by
// 99 KB of shared memory; this kernel follows CDNA4 instead:
//
//  * Operand tiles move HBM -> LDS with gfx950's direct global-to-LDS loads
//    (global_load_lds_dwordx4 / _dword): no staging registers, no LDS store
//    instructions.  Packed data stays packed in LDS (0.5625 B per element),
//    so a 256 x 128-element stage of both operands is 36 KB and a 3-deep ring
//    fits easily in the 160 KB LDS.  Rows are XOR-swizzled in 16-byte chunks
//    (the swizzle is applied by choosing each lane's source address, since a
//    direct load writes lane L at slot L) so fragment reads are conflict-free.
//  * Each wave dequantises its fragments in registers to fp16 -- exactly, as
//    E2M1 * E4M3 has at most 6 significant bits -- with one hardware FP4 ->
//    fp16 conversion and one packed fp16 multiply per element pair, and feeds
//    v_mfma_f32_32x32x16_f16 with fp32 accumulation.  Because the E4M3 factor
//    is applied to the operands, the 16-element blocks need no correction of
//    the accumulator.
//  * K is permuted inside a stage, identically for A and B (a contraction is
//    order-free): lane half g = lane / 32 owns stage elements [64g, 64g+64) of
//    its row and MFMA step t takes its dword t, so one 32-byte LDS read feeds
//    eight MFMA steps.
//  * Workgroup ids are regrouped XCD-aware: hardware ids go round-robin over
//    the 8 XCDs, so each XCD is given a compact block of output tiles whose
//    A and B rows it shares in its own L2.
#include "nvfp4_device.h"
#include "nvfp4_encode.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kBK = 128;        // K elements per stage
constexpr int kRowBytes = 64;   // nibble bytes per row per stage
constexpr int kScBytes = 8;     // scale bytes per row per stage
// Tuning knobs (compile-time): ring depth, row-swizzle shift, tile-row group.
#ifndef NVFP4_MFMA_STAGES
#define NVFP4_MFMA_STAGES 4
#endif
#ifndef NVFP4_MFMA_SWZ_SHIFT
#define NVFP4_MFMA_SWZ_SHIFT 1
#endif
#ifndef NVFP4_MFMA_GROUP_M
#define NVFP4_MFMA_GROUP_M 8
#endif
constexpr int kStages = NVFP4_MFMA_STAGES;  // LDS ring depth

template <int BM, int BN>
struct Smem {
  static constexpr int kANib = 0;
  static constexpr int kBNib = kANib + BM * kRowBytes;
  static constexpr int kASc = kBNib + BN * kRowBytes;
  static constexpr int kBSc = kASc + BM * kScBytes;
  static constexpr int kBytes = kBSc + BN * kScBytes;  // one stage
};

// Direct buffer loads into LDS.  Each lane reads `size` bytes at
// p + voff + soff (raw buffer, stride 0, range `bytes`: accesses past the end
// read as zero) and the wave writes them to lds + lane * size.  The
// descriptor is built from scalar values, so it stays in SGPRs.
__device__ __forceinline__ void buffer_load_lds16(const void* p, uint32_t bytes, void* lds,
                                                  uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000),
      (lds_void_ptr)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(const void* p, uint32_t bytes, void* lds,
                                                 uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000),
      (lds_void_ptr)lds, 4, voff, soff, 0, 0);
}

// 16-byte chunk swizzle of a 64-byte LDS row: physical chunk = logical ^ swz.
__device__ __forceinline__ int swz(int row) { return (row >> NVFP4_MFMA_SWZ_SHIFT) & 3; }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Workgroup barrier that is also a compiler memory barrier, without the
// full memory-counter drain __syncthreads() implies: the loads still in flight
// target other ring buffers, and each wave has already waited for its own
// loads of the stage about to be read.
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if ((nt & 7) == 0) pid = (pid & 7) * (nt >> 3) + (pid >> 3);
  constexpr int GROUP_M = NVFP4_MFMA_GROUP_M;
  const int per_group = GROUP_M * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// A wave's 32-row fragment of one stage, split by when it is consumed:
// `lo` (MFMA steps 0-3) and `hi` (steps 4-7), 16 bytes each, plus the
// lane's 4 E4M3 block scale bytes (converted to fp16 pairs only when first
// needed, so the LDS read latency is never waited on).
struct FragLo {
  u32x4 d;
  uint32_t s4;
};

__device__ __forceinline__ FragLo read_lo(const uint8_t* nib, const uint8_t* sc, int row, int g) {
  FragLo f;
  f.d = *reinterpret_cast<const u32x4*>(nib + row * kRowBytes + (((2 * g) ^ swz(row)) << 4));
  f.s4 = *reinterpret_cast<const uint32_t*>(sc + row * kScBytes + 4 * g);
  return f;
}

__device__ __forceinline__ u32x4 read_hi(const uint8_t* nib, int row, int g) {
  return *reinterpret_cast<const u32x4*>(nib + row * kRowBytes + (((2 * g + 1) ^ swz(row)) << 4));
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Cfg {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  static constexpr int FM = TM / 32, FN = TN / 32;
  // direct-load instructions per wave per stage
  static constexpr int kANibLoads = BM * kRowBytes / 1024 / kWaves;
  static constexpr int kBNibLoads = BN * kRowBytes / 1024 / kWaves;
  // scale loads (4 bytes per lane) of a whole stage; a tile with fewer
  // than one per wave gives every wave one, the extra waves repeating one
  // exactly (identical bytes to the same LDS slot), so that every wave
  // issues the same number of loads and the fixed waits stay exact
  static constexpr int kAScTotal = BM * kScBytes / 256;
  static constexpr int kBScTotal = BN * kScBytes / 256;
  static constexpr int kAScLoads = kAScTotal >= kWaves ? kAScTotal / kWaves : 1;
  static constexpr int kBScLoads = kBScTotal >= kWaves ? kBScTotal / kWaves : 1;
  static constexpr int kLoads = kANibLoads + kBNibLoads + kAScLoads + kBScLoads;
  static_assert(kANibLoads >= 1 && kBNibLoads >= 1 && kAScTotal >= 1 && kBScTotal >= 1,
                "tile too small for the load split");
  static_assert((kAScTotal < kWaves || kAScTotal % kWaves == 0) &&
                    (kBScTotal < kWaves || kBScTotal % kWaves == 0),
                "scale loads split evenly over the waves");
  // first scale-load slot of wave w
  static __device__ __forceinline__ int asc_slot(int w) {
    return kAScTotal >= kWaves ? w * kAScLoads : w % kAScTotal;
  }
  static __device__ __forceinline__ int bsc_slot(int w) {
    return kBScTotal >= kWaves ? w * kBScLoads : w % kBScTotal;
  }
};

// Output tile writer.  acc[i][j] register r holds row 8*(r/4) + 4*(lane/32)
// + r%4, column lane%32 of its 32x32 tile (row0 / col0: the wave's origin).
// Whole tiles of an output under 4 GiB have no per-element branches:
//  * bf16 with 16-byte aligned rows: the wave converts its tile (pairs of
//    rows in one instruction, round to nearest even) into its own region of
//    the now idle LDS, reads it back by rows and writes 16 bytes per lane, so
//    every store fills whole cache lines;
//  * otherwise buffer stores of single elements, the row offset in a scalar
//    register and the lane's column offset fixed.
// Edge tiles check every element.
template <int DT, int FM, int FN>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], float alpha, void* y,
                                           int64_t ld_y, int M, int N, int row0, int col0,
                                           int lane, bool whole, bool vec, uint32_t y_bytes,
                                           uint8_t* region) {
  constexpr int ES = DT == 0 ? 4 : 2;
  constexpr int TM = FM * 32, TN = FN * 32;
  const int lg = lane >> 5, li = lane & 31;
  if (whole && DT == 1 && vec) {
    constexpr int RS = TN * 2 + 16;  // padded LDS row stride (bytes)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t b = __builtin_bit_cast(
              uint32_t, __builtin_convertvector(f32x2{acc[i][j][r] * alpha, acc[i][j][r + 1] * alpha}, bf16x2));
          uint8_t* p = region + row * RS + (j * 32 + li) * 2;
          *reinterpret_cast<uint16_t*>(p) = (uint16_t)b;
          *reinterpret_cast<uint16_t*>(p + RS) = (uint16_t)(b >> 16);
        }
      }
    // LDS accesses of one wave complete in order: the reads below see the
    // writes above
    constexpr int LPR = TN / 8;            // lanes per row (16 bytes each)
    constexpr int RPI = 64 / LPR;          // rows per instruction
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(y, (short)0, (int)y_bytes, 0x00020000);
    const int lr = lane / LPR, lc = lane % LPR;
    const uint32_t voff = (uint32_t)(lr * ld_y + lc * 8) * 2;
#pragma unroll
    for (int p = 0; p < TM / RPI; ++p) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + (p * RPI + lr) * RS + lc * 16);
      const uint32_t soff = ((uint32_t)(row0 + p * RPI) * (uint32_t)ld_y + (uint32_t)col0) * 2;
      __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, voff, soff, 0);
    }
  } else if (whole) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(y, (short)0, (int)y_bytes, 0x00020000);
    const uint32_t lane_off = (uint32_t)((4 * lg) * ld_y + li) * ES;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t row = (uint32_t)(row0 + i * 32 + 8 * (r >> 2) + (r & 3));
        const uint32_t s0 = (row * (uint32_t)ld_y + (uint32_t)col0) * ES;
        const uint32_t s1 = s0 + (uint32_t)ld_y * ES;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float v0 = acc[i][j][r] * alpha, v1 = acc[i][j][r + 1] * alpha;
          if constexpr (DT == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v0), rsrc, lane_off + j * 32 * ES, s0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v1), rsrc, lane_off + j * 32 * ES, s1, 0);
          } else {
            const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v0, v1}, bf16x2));
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b, rsrc, lane_off + j * 32 * ES, s0, 0);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(b >> 16), rsrc, lane_off + j * 32 * ES, s1, 0);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 32 + li;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (row < M && col < N) store_out(y, (int64_t)row * ld_y + col, acc[i][j][r] * alpha, DT);
        }
      }
  }
}

// NVFP4 output tile: the fp32 values fl32(alpha * acc) that the fp32 writer
// would store are staged by rows in the wave's LDS region (half the wave
// tile per pass), and each lane then encodes whole 16-column blocks with the
// quantiser's exact block encoder, given the output's global scale.
template <int kMode, int FM, int FN>
__device__ __forceinline__ void quant_tile(const f32x16 (&acc)[FM][FN], float alpha, int M, int N,
                                           int row0, int col0, int lane, uint8_t* region,
                                           const QuantOut& qo, const enc::EncodeParams& P) {
  constexpr int TN = FN * 32;
  constexpr int PF = FM >= 2 ? FM / 2 : 1;  // fragment rows per pass
  constexpr int PR = PF * 32;               // tile rows per pass
  constexpr int RS = TN * 4 + 16;           // padded LDS row stride (bytes)
  constexpr int BPR = TN / 16;              // 16-column blocks per row
  constexpr int NB = PR * BPR;              // blocks per pass
  static_assert(NB % 64 == 0, "whole blocks per lane");
  const int lg = lane >> 5, li = lane & 31;
  const int64_t qld = N / 2, sld = N / 16;
#pragma unroll
  for (int pass = 0; pass < FM / PF; ++pass) {
#pragma unroll
    for (int i = 0; i < PF; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
          *reinterpret_cast<float*>(region + row * RS + (j * 32 + li) * 4) =
              acc[pass * PF + i][j][r] * alpha;
        }
    // LDS accesses of one wave complete in order: the reads below see the
    // writes above, and the next pass's writes follow these reads
    // blocks in groups of up to four: all of a group's LDS reads go out
    // before its first encode, so the four encodes overlap each other's
    // latency instead of each waiting on its own reads
    constexpr int NT = NB / 64, GB = NT < 4 ? NT : 4;
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += GB) {
      enc::Block16 b[GB];
#pragma unroll
      for (int u = 0; u < GB; ++u) {
        const int blk = (t0 + u) * 64 + lane, row = blk / BPR, cb = blk % BPR;
        const u32x4* src = reinterpret_cast<const u32x4*>(region + row * RS + cb * 64);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x4 v = src[w];
#pragma unroll
          for (int e = 0; e < 4; ++e) b[u].v[4 * w + e] = __uint_as_float(v[e]);
        }
      }
#pragma unroll
      for (int u = 0; u < GB; ++u) {
        const int blk = (t0 + u) * 64 + lane, row = blk / BPR, cb = blk % BPR;
        const int grow = row0 + pass * PR + row, gcol = col0 + cb * 16;
        if (grow < M && gcol < N)
          enc::encode_block<kMode>(b[u], P, qo.q + (int64_t)grow * qld + gcol / 2,
                                   qo.s + (int64_t)grow * sld + gcol / 16);
      }
    }
  }
}

// Stage variants of the main loop (4-deep ring):
//   kFull  - mid-stage sync waits for stage s+1 with one younger stage in
//            flight, then refills the ring with stage s+3;
//   kTail1 - same wait, nothing left to load;
//   kTail0 - stage s+1 is the youngest load: wait for all;
//   kLast  - no next stage.
enum StageMode { kFull, kTail1, kTail0, kLast };

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_mfma_kernel(
    int M, int N, int K, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y, uint32_t y_bytes, int y_flags, QuantOut qo) {
  static_assert(kStages == 4, "stage modes assume a 4-deep ring");
  using C = Cfg<BM, BN, WAVES_M, WAVES_N>;
  using L = Smem<BM, BN>;
  constexpr int FM = C::FM, FN = C::FN, NF = FM + FN, Q = FM * FN;
  constexpr int P = 2 * NF;  // dequant pieces per MFMA step
  static_assert(NF <= 2 * Q, "the lo reads of a stage fit in the MFMAs of steps 3 and 4");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar, so LDS destinations (M0) are scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int li = lane & 31, lg = lane >> 5;

  int tm, tn;
  tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t rowq = (uint32_t)(K / 2), rows = (uint32_t)(K / 16);
  const int nstage = K / kBK;

  // Per-lane 32-bit source offsets (operands are < 4 GiB; checked by the
  // launcher) relative to the stage's column origin.  Rows past M / N are
  // clamped to the last valid row: they only feed outputs that are not stored.
  uint32_t a_nib_off[C::kANibLoads], b_nib_off[C::kBNibLoads];
  uint32_t a_sc_off[C::kAScLoads], b_sc_off[C::kBScLoads];
#pragma unroll
  for (int i = 0; i < C::kANibLoads; ++i) {
    const int slot = (wave * C::kANibLoads + i) * 64 + lane;   // 16-byte LDS slot
    const int r = slot >> 2, phys = slot & 3;
    a_nib_off[i] = (uint32_t)min(m0 + r, M - 1) * rowq + ((phys ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::kBNibLoads; ++i) {
    const int slot = (wave * C::kBNibLoads + i) * 64 + lane;
    const int r = slot >> 2, phys = slot & 3;
    b_nib_off[i] = (uint32_t)min(n0 + r, N - 1) * rowq + ((phys ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::kAScLoads; ++i) {
    const int slot = (C::asc_slot(wave) + i) * 64 + lane;        // 4-byte LDS slot
    a_sc_off[i] = (uint32_t)min(m0 + (slot >> 1), M - 1) * rows + ((slot & 1) << 2);
  }
#pragma unroll
  for (int i = 0; i < C::kBScLoads; ++i) {
    const int slot = (C::bsc_slot(wave) + i) * 64 + lane;
    b_sc_off[i] = (uint32_t)min(n0 + (slot >> 1), N - 1) * rows + ((slot & 1) << 2);
  }

  // Byte ranges of the four operand arrays (< 4 GiB, checked by the launcher).
  // The per-lane offsets above stay in VGPRs for the whole kernel and the
  // stage's column offset is a scalar operand, so a direct load costs no
  // vector instructions.
  const uint32_t aq_bytes = (uint32_t)M * rowq, bq_bytes = (uint32_t)N * rowq;
  const uint32_t as_bytes = (uint32_t)M * rows, bs_bytes = (uint32_t)N * rows;

  // Direct load number J (0 .. kLoads-1) of stage st into its ring buffer.
  auto load_one = [&](int st, auto jc) {
    constexpr int J = decltype(jc)::value;
    uint8_t* base = smem + (st & (kStages - 1)) * L::kBytes;
    if constexpr (J < C::kANibLoads) {
      buffer_load_lds16(a_q, aq_bytes, base + L::kANib + (wave * C::kANibLoads + J) * 1024,
                        a_nib_off[J], (uint32_t)st * kRowBytes);
    } else if constexpr (J < C::kANibLoads + C::kBNibLoads) {
      constexpr int i = J - C::kANibLoads;
      buffer_load_lds16(b_q, bq_bytes, base + L::kBNib + (wave * C::kBNibLoads + i) * 1024,
                        b_nib_off[i], (uint32_t)st * kRowBytes);
    } else if constexpr (J < C::kANibLoads + C::kBNibLoads + C::kAScLoads) {
      constexpr int i = J - C::kANibLoads - C::kBNibLoads;
      buffer_load_lds4(a_s, as_bytes, base + L::kASc + (C::asc_slot(wave) + i) * 256,
                       a_sc_off[i], (uint32_t)st * kScBytes);
    } else {
      constexpr int i = J - C::kANibLoads - C::kBNibLoads - C::kAScLoads;
      buffer_load_lds4(b_s, bs_bytes, base + L::kBSc + (C::bsc_slot(wave) + i) * 256,
                       b_sc_off[i], (uint32_t)st * kScBytes);
    }
  };
  auto issue = [&](int st) { static_for<C::kLoads>([&](auto jc) { load_one(st, jc); }); };

  auto frag_row = [&](int f) { return f < FM ? wm * C::TM + f * 32 + li : wn * C::TN + (f - FM) * 32 + li; };
  auto nib_base = [&](int st, int f) {
    return smem + (st & (kStages - 1)) * L::kBytes + (f < FM ? L::kANib : L::kBNib);
  };
  auto sc_base = [&](int st, int f) {
    return smem + (st & (kStages - 1)) * L::kBytes + (f < FM ? L::kASc : L::kBSc);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  FragLo lo[NF];
  u32x4 hi[NF];
  Scales sc[NF];
  f16x8 cur[NF];

  // ---- prologue: stages 0..2 in flight, stage 0 read, step 0 dequantised
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < nstage) issue(st);
  if (nstage >= 3) wait_vmcnt<2 * C::kLoads>();
  else if (nstage == 2) wait_vmcnt<C::kLoads>();
  else wait_vmcnt<0>();
  workgroup_barrier();
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    lo[f] = read_lo(nib_base(0, f), sc_base(0, f), frag_row(f), lg);
    hi[f] = read_hi(nib_base(0, f), frag_row(f), lg);
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    sc[f] = to_scales(lo[f].s4);
    dequant_piece<0, 0>(lo[f].d[0], sc[f], cur[f]);
    dequant_piece<0, 1>(lo[f].d[0], sc[f], cur[f]);
  }

  // ---- one stage: 8 MFMA steps of FM x FN 32x32x16 MFMAs.  After each MFMA
  // of step T go the dequant pieces of step T+1 (P pieces spread over the Q
  // MFMAs), so the matrix core never waits on a long run of vector ops.
  // Between steps 2 and 3 the workgroup syncs on stage s+1 (its `lo` halves
  // are dead by then); step 3 reads them into registers and refills the ring;
  // step 7 reads the `hi` halves of s+1 and dequantises its step 0.
  auto run_stage = [&](int s, auto mc) {
    constexpr StageMode MODE = decltype(mc)::value;
    constexpr bool NEXT = MODE != kLast;
    FragLo nlo[NF];
    u32x4 nhi[NF];
    Scales nsc[NF];
    f16x8 nxt[NF];
    static_for<8>([&](auto tc) {
      constexpr int T = decltype(tc)::value;
      if constexpr (T == 3 && NEXT) {
        if constexpr (MODE == kTail0) wait_vmcnt<0>();
        else wait_vmcnt<C::kLoads>();
        workgroup_barrier();
      }
      static_for<Q>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        constexpr int i = I / FN, j = I % FN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[i], cur[FM + j], acc[i][j], 0, 0, 0);
        // dequant pieces [I*P/Q, (I+1)*P/Q) of the next step
        static_for<(I + 1) * P / Q - I * P / Q>([&](auto pc) {
          constexpr int p = I * P / Q + decltype(pc)::value;
          constexpr int F = p / 2, H = p % 2;
          if constexpr (T < 3) {
            dequant_piece<T + 1, H>(lo[F].d[T + 1], sc[F], nxt[F]);
          } else if constexpr (T < 7) {
            dequant_piece<T + 1, H>(hi[F][T - 3], sc[F], nxt[F]);
          } else if constexpr (NEXT) {
            if constexpr (H == 0) nsc[F] = to_scales(nlo[F].s4);
            dequant_piece<0, H>(nlo[F].d[0], nsc[F], nxt[F]);
          }
        });
        if constexpr ((T == 3 || T == 4) && NEXT) {
          // lo halves of stage s+1 into registers over the 2Q MFMAs of steps
          // 3 and 4: one fragment every other MFMA, or every MFMA when a step
          // has fewer MFMAs than fragments
          constexpr int SL = (T - 3) * Q + I;
          if constexpr (NF <= Q) {
            if constexpr (SL % 2 == 0 && SL / 2 < NF)
              nlo[SL / 2] = read_lo(nib_base(s + 1, SL / 2), sc_base(s + 1, SL / 2), frag_row(SL / 2), lg);
          } else if constexpr (SL < NF) {
            nlo[SL] = read_lo(nib_base(s + 1, SL), sc_base(s + 1, SL), frag_row(SL), lg);
          }
        }
        if constexpr (T >= 3 && T <= 6 && MODE == kFull) {
          // refill the ring: the kLoads direct loads spread over steps 3-6
          constexpr int SL = (T - 3) * Q + I, NS = 4 * Q;
          constexpr int J0 = SL * C::kLoads / NS, J1 = (SL + 1) * C::kLoads / NS;
          static_for<J1 - J0>([&](auto jc) {
            load_one(s + kStages - 1, std::integral_constant<int, J0 + decltype(jc)::value>{});
          });
        }
        if constexpr (T == 7 && NEXT) {
          // hi halves of stage s+1: fragments I, I + Q, ... at MFMA I
          static_for<(NF + Q - 1) / Q>([&](auto kc) {
            constexpr int F = I + decltype(kc)::value * Q;
            if constexpr (F < NF) nhi[F] = read_hi(nib_base(s + 1, F), frag_row(F), lg);
          });
        }
        // the hi reads of the previous stage finished long ago; saying so
        // here keeps the compiler from waiting for them behind newer reads
        if constexpr (T == 0 && I == 0) wait_lgkmcnt0();
        // likewise for the lo reads of step 3, before step 7 issues new reads
        if constexpr (T == 6 && I == 0 && NEXT) wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (T < 7 || NEXT) {
#pragma unroll
        for (int f = 0; f < NF; ++f) cur[f] = nxt[f];
      }
    });
    if constexpr (NEXT) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        lo[f] = nlo[f];
        hi[f] = nhi[f];
        sc[f] = nsc[f];
      }
    }
  };

  int s = 0;
  for (; s + kStages - 1 < nstage; ++s) run_stage(s, std::integral_constant<StageMode, kFull>{});
  if (s + 2 < nstage) run_stage(s++, std::integral_constant<StageMode, kTail1>{});
  if (s + 1 < nstage) run_stage(s++, std::integral_constant<StageMode, kTail0>{});
  run_stage(s, std::integral_constant<StageMode, kLast>{});

  // ---- epilogue: y = fl32(ga * gb) * acc.  The ring is idle once every
  // wave has finished its last stage; each wave then owns a region of it.
  const float alpha = a_g[0] * b_g[0];
  const bool whole = y_bytes != 0 && m0 + BM <= M && n0 + BN <= N;
  const bool vec = (y_flags & 1) != 0;
  const int row0 = m0 + wm * C::TM, col0 = n0 + wn * C::TN;
  // a wave's staging region: its bf16 tile, or half its fp32 tile (a
  // 32-row fp32 pass when the tile is 32 rows tall) for the NVFP4 encoder
  constexpr int kRegionBf16 = C::TM * (C::TN * 2 + 16);
  constexpr int kRegionQuant = (C::FM >= 2 ? C::FM / 2 : 1) * 32 * (C::TN * 4 + 16);
  constexpr int kRegion = kRegionBf16 > kRegionQuant ? kRegionBf16 : kRegionQuant;
  static_assert(C::kWaves * kRegion <= kStages * L::kBytes, "epilogue staging exceeds the ring");
  workgroup_barrier();
  uint8_t* region = smem + wave * kRegion;
  // the lane index again, from the hardware lane counter: an expression the
  // compiler cannot equate with the one before the main loop, so nothing
  // lane-dependent has to stay live (or spill) across the loop for this
  const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if (y_dtype == 2) {
    static_assert((C::FM >= 2 ? C::FM / 2 : 1) * 32 * (C::TN * 4 + 16) <= kRegion,
                  "quantising epilogue staging exceeds the wave's region");
    const float g = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(qo.g[0])));
    const enc::EncodeParams P = enc::make_params(g);
    const int mode = enc::encode_mode(g);
    if (mode == 1) quant_tile<1>(acc, alpha, M, N, row0, col0, elane, region, qo, P);
    else if (mode == 0) quant_tile<0>(acc, alpha, M, N, row0, col0, elane, region, qo, P);
    else quant_tile<2>(acc, alpha, M, N, row0, col0, elane, region, qo, P);
  } else if (y_dtype == 0) {
    store_tile<0>(acc, alpha, y, ld_y, M, N, row0, col0, elane, whole, vec, y_bytes, region);
  } else {
    store_tile<1>(acc, alpha, y, ld_y, M, N, row0, col0, elane, whole, vec, y_bytes, region);
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_cfg(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                      void* y, int y_dtype, int64_t ld_y, hipStream_t stream, QuantOut qo) {
  using L = Smem<BM, BN>;
  using C = Cfg<BM, BN, WAVES_M, WAVES_N>;
  const int smem = kStages * L::kBytes;
  auto kern = gemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N>;
  // once per process (thread-safe static initialisation)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // extent of y in bytes when below 4 GiB (whole tiles then use 32-bit
  // buffer offsets), else 0 (every tile takes the checked writer)
  const int64_t extent = y_dtype == 2 ? 0 : ((M - 1) * ld_y + N) * (y_dtype == 0 ? 4 : 2);
  const uint32_t y_bytes = extent < (int64_t)0xFFFFFFFF ? (uint32_t)extent : 0u;
  // bit 0: rows start on 16-byte boundaries (16-byte stores of bf16 rows)
  const int y_flags = ((reinterpret_cast<uintptr_t>(y) & 15) == 0 && ld_y % 8 == 0) ? 1 : 0;
  kern<<<(unsigned)tiles, C::kThreads, smem, stream>>>((int)M, (int)N, (int)K, a.q, a.s, a.g,
                                                        b.q, b.s, b.g, y, y_dtype, ld_y, y_bytes,
                                                        y_flags, qo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP4 GEMM on the scaled FP4 matrix instruction.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1 multiplies a
// 32 x 64 by a 64 x 32 fragment of packed nibbles and applies one E8M0
// scale per lane: lane L holds row (or column) L % 32 and 32 consecutive
// K-elements, exactly one 32-element block, plus that block's scale byte
// (checked against an exact product on every lane).  No dequantisation is
// left to the vector unit, so the kernel is the same LDS ring as above with
// the products issued straight from the fragment reads:
//  * a stage is 128 K-elements: 64 bytes of nibbles and 4 scale bytes per
//    row, moved HBM -> LDS by direct loads into a 4-deep ring, rows XOR-
//    swizzled in 16-byte chunks as above;
//  * K is permuted inside a stage (identically for both operands): lane
//    half g owns blocks 2g and 2g + 1 of the stage, so MFMA step t (0, 1)
//    reads 16-byte chunk 2g + t of its row and scale byte t of the two it
//    loads at once;
//  * per stage: step 0's products run while the step-1 fragments are read
//    and the ring is refilled; the workgroup then syncs on stage s + 1, and
//    step 1's products run while stage s + 1's step-0 fragments are read.
//    Every stage issues the same loads (past the last stage a harmless
//    reload of it into a slot no stage reads again), so the waits are fixed.
constexpr int kMxScBytes = 4;   // E8M0 bytes per row per stage (128 / 32)

template <int BM, int BN>
struct SmemMx {
  static constexpr int kANib = 0;
  static constexpr int kBNib = kANib + BM * kRowBytes;
  static constexpr int kASc = kBNib + BN * kRowBytes;
  static constexpr int kBSc = kASc + BM * kMxScBytes;
  static constexpr int kBytes = kBSc + BN * kMxScBytes;  // one stage
};

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct CfgMx {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int kANibLoads = BM * kRowBytes / 1024 / kWaves;
  static constexpr int kBNibLoads = BN * kRowBytes / 1024 / kWaves;
  // scale loads (4 bytes per lane, 256 bytes per instruction); with fewer
  // than one per wave the extra waves repeat one exactly (same bytes to the
  // same LDS slot), so every wave issues the same number of loads
  static constexpr int kAScTotal = (BM * kMxScBytes + 255) / 256;
  static constexpr int kBScTotal = (BN * kMxScBytes + 255) / 256;
  static constexpr int kAScLoads = kAScTotal >= kWaves ? kAScTotal / kWaves : 1;
  static constexpr int kBScLoads = kBScTotal >= kWaves ? kBScTotal / kWaves : 1;
  static constexpr int kLoads = kANibLoads + kBNibLoads + kAScLoads + kBScLoads;
  static_assert(kANibLoads >= 1 && kBNibLoads >= 1, "tile too small for the load split");
  static_assert(BM * kMxScBytes % 256 == 0 && BN * kMxScBytes % 256 == 0,
                "whole scale-load instructions");
  static_assert((kAScTotal < kWaves || kAScTotal % kWaves == 0) &&
                    (kBScTotal < kWaves || kBScTotal % kWaves == 0),
                "scale loads split evenly over the waves");
  static __device__ __forceinline__ int asc_slot(int w) {
    return kAScTotal >= kWaves ? w * kAScLoads : w % kAScTotal;
  }
  static __device__ __forceinline__ int bsc_slot(int w) {
    return kBScTotal >= kWaves ? w * kBScLoads : w % kBScTotal;
  }
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// 16-byte fragment chunk of step t for lane half g (rows XOR-swizzled).
__device__ __forceinline__ u32x4 read_mx_chunk(const uint8_t* nib, int row, int g, int t) {
  return *reinterpret_cast<const u32x4*>(nib + row * kRowBytes + (((2 * g + t) ^ swz(row)) << 4));
}

// Scale bytes of blocks 2g, 2g + 1 of the lane's row: byte t is step t's.
__device__ __forceinline__ uint32_t read_mx_scales(const uint8_t* sc, int row, int g) {
  return *reinterpret_cast<const uint16_t*>(sc + row * kMxScBytes + 2 * g);
}

template <int T>
__device__ __forceinline__ f32x16 mx_mfma(const u32x4& a, uint32_t sa, const u32x4& b,
                                          uint32_t sb, const f32x16& c) {
  // E2M1 operands (format code 4) occupy the first four registers
  const i32x8 a8 = __builtin_shufflevector(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, a),
                                           0, 1, 2, 3, 0, 1, 2, 3);
  const i32x8 b8 = __builtin_shufflevector(__builtin_bit_cast(i32x4, b), __builtin_bit_cast(i32x4, b),
                                           0, 1, 2, 3, 0, 1, 2, 3);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, T, (int)sa, T, (int)sb);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_mx_kernel(
    int M, int N, int K, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s, void* __restrict__ y,
    int y_dtype, int64_t ld_y, uint32_t y_bytes, int y_flags) {
  static_assert(kStages == 4, "the ring is 4 deep");
  using C = CfgMx<BM, BN, WAVES_M, WAVES_N>;
  using L = SmemMx<BM, BN>;
  constexpr int FM = C::FM, FN = C::FN, NF = FM + FN;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int li = lane & 31, lg = lane >> 5;

  int tm, tn;
  tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t rowq = (uint32_t)(K / 2), rows = (uint32_t)(K / 32);
  const int nstage = K / kBK;

  // per-lane source offsets (rows past M / N clamped to the last row: they
  // only feed outputs that are not stored)
  uint32_t a_nib_off[C::kANibLoads], b_nib_off[C::kBNibLoads];
  uint32_t a_sc_off[C::kAScLoads], b_sc_off[C::kBScLoads];
#pragma unroll
  for (int i = 0; i < C::kANibLoads; ++i) {
    const int slot = (wave * C::kANibLoads + i) * 64 + lane;
    const int r = slot >> 2, phys = slot & 3;
    a_nib_off[i] = (uint32_t)min(m0 + r, M - 1) * rowq + ((phys ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::kBNibLoads; ++i) {
    const int slot = (wave * C::kBNibLoads + i) * 64 + lane;
    const int r = slot >> 2, phys = slot & 3;
    b_nib_off[i] = (uint32_t)min(n0 + r, N - 1) * rowq + ((phys ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::kAScLoads; ++i) {
    const int slot = (C::asc_slot(wave) + i) * 64 + lane;  // 4-byte slot = one row
    a_sc_off[i] = (uint32_t)min(m0 + slot, M - 1) * rows;
  }
#pragma unroll
  for (int i = 0; i < C::kBScLoads; ++i) {
    const int slot = (C::bsc_slot(wave) + i) * 64 + lane;
    b_sc_off[i] = (uint32_t)min(n0 + slot, N - 1) * rows;
  }
  const uint32_t aq_bytes = (uint32_t)M * rowq, bq_bytes = (uint32_t)N * rowq;
  const uint32_t as_bytes = (uint32_t)M * rows, bs_bytes = (uint32_t)N * rows;

  // the loads of stage st into ring slot `slot` (st past the end reloads
  // the last stage)
  auto issue = [&](int st, int slot) {
    const int src = min(st, nstage - 1);
    uint8_t* base = smem + slot * L::kBytes;
#pragma unroll
    for (int i = 0; i < C::kANibLoads; ++i)
      buffer_load_lds16(a_q, aq_bytes, base + L::kANib + (wave * C::kANibLoads + i) * 1024,
                        a_nib_off[i], (uint32_t)src * kRowBytes);
#pragma unroll
    for (int i = 0; i < C::kBNibLoads; ++i)
      buffer_load_lds16(b_q, bq_bytes, base + L::kBNib + (wave * C::kBNibLoads + i) * 1024,
                        b_nib_off[i], (uint32_t)src * kRowBytes);
#pragma unroll
    for (int i = 0; i < C::kAScLoads; ++i)
      buffer_load_lds4(a_s, as_bytes, base + L::kASc + (C::asc_slot(wave) + i) * 256,
                       a_sc_off[i], (uint32_t)src * kMxScBytes);
#pragma unroll
    for (int i = 0; i < C::kBScLoads; ++i)
      buffer_load_lds4(b_s, bs_bytes, base + L::kBSc + (C::bsc_slot(wave) + i) * 256,
                       b_sc_off[i], (uint32_t)src * kMxScBytes);
  };

  auto frag_row = [&](int f) { return f < FM ? wm * C::TM + f * 32 + li : wn * C::TN + (f - FM) * 32 + li; };
  auto nib_base = [&](int st, int f) {
    return smem + (st & (kStages - 1)) * L::kBytes + (f < FM ? L::kANib : L::kBNib);
  };
  auto sc_base = [&](int st, int f) {
    return smem + (st & (kStages - 1)) * L::kBytes + (f < FM ? L::kASc : L::kBSc);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  u32x4 f0[NF], f1[NF];  // step 0 / step 1 fragments of the current stage
  uint32_t sc[NF];       // their scale pairs

  // prologue: stages 0..2 in flight, stage 0's step-0 fragments read
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st) issue(st, st);
  wait_vmcnt<2 * C::kLoads>();
  workgroup_barrier();
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    f0[f] = read_mx_chunk(nib_base(0, f), frag_row(f), lg, 0);
    sc[f] = read_mx_scales(sc_base(0, f), frag_row(f), lg);
  }

  constexpr int Q = FM * FN;                  // products per step
  constexpr int kIssueAt = NF < Q - 1 ? NF : Q - 1;  // product after which the refill goes
  for (int s = 0; s < nstage; ++s) {
    wait_lgkmcnt0();  // stage s's step-0 fragments
    // step 0: products of f0 while f1 is read and the ring is refilled
    static_for<Q>([&](auto ic) {
      constexpr int I = decltype(ic)::value, i = I / FN, j = I % FN;
      acc[i][j] = mx_mfma<0>(f0[i], sc[i], f0[FM + j], sc[FM + j], acc[i][j]);
      if constexpr (I < NF) f1[I] = read_mx_chunk(nib_base(s, I), frag_row(I), lg, 1);
      if constexpr (I == kIssueAt) issue(s + kStages - 1, (s + kStages - 1) & (kStages - 1));
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<(NF > Q ? NF - Q : 0)>([&](auto ic) {
      constexpr int I = Q + decltype(ic)::value;
      f1[I] = read_mx_chunk(nib_base(s, I), frag_row(I), lg, 1);
    });
    // the step-1 fragments are in registers and this wave's loads of stage
    // s + 1 have landed; after the barrier every wave's have, and every
    // wave is done reading stage s - 1 (whose slot the refill above took)
    wait_lgkmcnt0();
    wait_vmcnt<2 * C::kLoads>();
    workgroup_barrier();
    // step 1: products of f1 while stage s + 1's step-0 fragments are read
    const bool next = s + 1 < nstage;
    uint32_t nsc[NF];
    static_for<Q>([&](auto ic) {
      constexpr int I = decltype(ic)::value, i = I / FN, j = I % FN;
      acc[i][j] = mx_mfma<1>(f1[i], sc[i], f1[FM + j], sc[FM + j], acc[i][j]);
      if constexpr (I < NF) {
        if (next) {
          f0[I] = read_mx_chunk(nib_base(s + 1, I), frag_row(I), lg, 0);
          nsc[I] = read_mx_scales(sc_base(s + 1, I), frag_row(I), lg);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<(NF > Q ? NF - Q : 0)>([&](auto ic) {
      constexpr int I = Q + decltype(ic)::value;
      if (next) {
        f0[I] = read_mx_chunk(nib_base(s + 1, I), frag_row(I), lg, 0);
        nsc[I] = read_mx_scales(sc_base(s + 1, I), frag_row(I), lg);
      }
    });
    if (next) {
#pragma unroll
      for (int f = 0; f < NF; ++f) sc[f] = nsc[f];
    }
  }

  // epilogue: the ring's last (padding) loads land, then each wave stages
  // its tile in its own region of the idle ring
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  const bool whole = y_bytes != 0 && m0 + BM <= M && n0 + BN <= N;
  const bool vec = (y_flags & 1) != 0;
  const int row0 = m0 + wm * C::TM, col0 = n0 + wn * C::TN;
  constexpr int kRegion = C::TM * (C::TN * 2 + 16);
  static_assert(C::kWaves * kRegion <= kStages * L::kBytes, "epilogue staging exceeds the ring");
  workgroup_barrier();
  uint8_t* region = smem + wave * kRegion;
  if (y_dtype == 0)
    store_tile<0>(acc, 1.0f, y, ld_y, M, N, row0, col0, lane, whole, vec, y_bytes, region);
  else
    store_tile<1>(acc, 1.0f, y, ld_y, M, N, row0, col0, lane, whole, vec, y_bytes, region);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_mx_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
                         const uint8_t* b_q, const uint8_t* b_s, void* y, int y_dtype,
                         int64_t ld_y, hipStream_t stream) {
  using L = SmemMx<BM, BN>;
  using C = CfgMx<BM, BN, WAVES_M, WAVES_N>;
  const int smem = kStages * L::kBytes;
  auto kern = gemm_mx_kernel<BM, BN, WAVES_M, WAVES_N>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t extent = ((M - 1) * ld_y + N) * (y_dtype == 0 ? 4 : 2);
  const uint32_t y_bytes = extent < (int64_t)0xFFFFFFFF ? (uint32_t)extent : 0u;
  const int y_flags = ((reinterpret_cast<uintptr_t>(y) & 15) == 0 && ld_y % 8 == 0) ? 1 : 0;
  kern<<<(unsigned)tiles, C::kThreads, smem, stream>>>((int)M, (int)N, (int)K, a_q, a_s, b_q, b_s,
                                                        y, y_dtype, ld_y, y_bytes, y_flags);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                            void* y, int y_dtype, int64_t ld_y, hipStream_t stream, QuantOut qo) {
  // The largest tile that still fills the chip for at least one round (the
  // larger the tile, the fewer dequantisations per MFMA): 256 x 256, then
  // 256 x 128, then 128 x 128 (4x the workgroups of 256 x 256).  Below that,
  // smaller tiles keep every CU busy and move fewer operand bytes per CU:
  // 128 x 64 while it fits one round (else one round of 128 x 128), then
  // 64 x 64 while that fits one round.
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (M >= 256 && N >= 256 && tiles(256, 256) >= 256)
    return launch_cfg<256, 256, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
  if (M >= 256 && N >= 128 && tiles(256, 128) >= 256)
    return launch_cfg<256, 128, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
  if (tiles(128, 128) >= 256 || tiles(128, 64) > 256)
    return launch_cfg<128, 128, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
  if (tiles(128, 64) == 256 || tiles(64, 64) > 256)
    return launch_cfg<128, 64, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
  return launch_cfg<64, 64, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
}

hipError_t launch_gemm_mx_mfma(int64_t M, int64_t N, int64_t K, const uint8_t* a_q,
                               const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                               void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
  // the same tile ladder as the NVFP4 kernel
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (M >= 256 && N >= 256 && tiles(256, 256) >= 256)
    return launch_mx_cfg<256, 256, 2, 2>(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype, ld_y, stream);
  if (M >= 256 && N >= 128 && tiles(256, 128) >= 256)
    return launch_mx_cfg<256, 128, 2, 2>(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype, ld_y, stream);
  if (tiles(128, 128) >= 256 || tiles(128, 64) > 256)
    return launch_mx_cfg<128, 128, 2, 2>(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype, ld_y, stream);
  return launch_mx_cfg<64, 64, 2, 2>(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype, ld_y, stream);
}

}  // namespace nvfp4
