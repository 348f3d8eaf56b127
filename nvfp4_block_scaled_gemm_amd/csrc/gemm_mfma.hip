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
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;

constexpr int kBK = 128;        // K elements per stage
constexpr int kRowBytes = 64;   // nibble bytes per row per stage
constexpr int kScBytes = 8;     // scale bytes per row per stage
constexpr int kStages = 3;      // LDS ring depth

template <int BM, int BN>
struct Smem {
  static constexpr int kANib = 0;
  static constexpr int kBNib = kANib + BM * kRowBytes;
  static constexpr int kASc = kBNib + BN * kRowBytes;
  static constexpr int kBSc = kASc + BM * kScBytes;
  static constexpr int kBytes = kBSc + BN * kScBytes;  // one stage
};

// 16-byte chunk swizzle of a 64-byte LDS row: physical chunk = logical ^ swz.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// 8 elements E2M1(nibble) * S from one packed dword, S a half of `sc`:
// the hardware converts each byte into two fp16 (low nibble first) and one
// packed multiply per pair applies S (selected half broadcast to both lanes).
template <int HALF>
__device__ __forceinline__ f16x8 dequant8(uint32_t packed, f16x2 sc) {
  const f16x2 s2 = __builtin_shufflevector(sc, sc, HALF, HALF);
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0) * s2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1) * s2;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2) * s2;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3) * s2;
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                 5, 6, 7);
}

// One wave-fragment of 32 rows for a stage: 32 nibble bytes + 4 scale bytes.
struct Frag {
  u32x4 lo, hi;    // dwords 0..3 and 4..7 (MFMA steps t = 0..7)
  f16x2 s01, s23;  // E4M3 scales of the lane's 4 blocks as fp16 pairs
};

__device__ __forceinline__ Frag read_frag(const uint8_t* nib, const uint8_t* sc, int row, int g) {
  Frag f;
  const int sw = swz(row);
  f.lo = *reinterpret_cast<const u32x4*>(nib + row * kRowBytes + (((2 * g) ^ sw) << 4));
  f.hi = *reinterpret_cast<const u32x4*>(nib + row * kRowBytes + (((2 * g + 1) ^ sw) << 4));
  const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sc + row * kScBytes + 4 * g);
  f.s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, false);
  f.s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s4, 1.0f, true);
  return f;
}

template <int T>
__device__ __forceinline__ f16x8 frag_step(const Frag& f) {
  constexpr int D = T & 3;
  const uint32_t w = (T < 4) ? f.lo[D] : f.hi[D];
  // step T uses block T/2 of the lane: 0,1 -> s01, 2,3 -> s23
  if constexpr ((T >> 1) == 0) return dequant8<0>(w, f.s01);
  else if constexpr ((T >> 1) == 1) return dequant8<1>(w, f.s01);
  else if constexpr ((T >> 1) == 2) return dequant8<0>(w, f.s23);
  else return dequant8<1>(w, f.s23);
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
  static constexpr int kAScLoads = BM * kScBytes / 256 / kWaves;
  static constexpr int kBScLoads = BN * kScBytes / 256 / kWaves;
  static constexpr int kLoads = kANibLoads + kBNibLoads + kAScLoads + kBScLoads;
  static_assert(kANibLoads >= 1 && kBNibLoads >= 1 && kAScLoads >= 1 && kBScLoads >= 1,
                "tile too small for the load split");
};

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_mfma_kernel(
    int M, int N, int K, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y) {
  using C = Cfg<BM, BN, WAVES_M, WAVES_N>;
  using L = Smem<BM, BN>;
  constexpr int FM = C::FM, FN = C::FN;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int li = lane & 31, lg = lane >> 5;

  int tm, tn;
  tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowq = K / 2, rows = K / 16;
  const int nstage = K / kBK;

  // Per-lane source offsets (bytes, relative to the stage's column origin).
  // Rows past M / N are clamped to the last valid row: they only feed outputs
  // that are never stored.
  int64_t a_nib_off[C::kANibLoads], b_nib_off[C::kBNibLoads];
  int64_t a_sc_off[C::kAScLoads], b_sc_off[C::kBScLoads];
#pragma unroll
  for (int i = 0; i < C::kANibLoads; ++i) {
    const int slot = (wave * C::kANibLoads + i) * 64 + lane;   // 16-byte LDS slot
    const int r = slot >> 2, phys = slot & 3;
    const int gr = min(m0 + r, M - 1);
    a_nib_off[i] = (int64_t)gr * rowq + ((phys ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::kBNibLoads; ++i) {
    const int slot = (wave * C::kBNibLoads + i) * 64 + lane;
    const int r = slot >> 2, phys = slot & 3;
    const int gr = min(n0 + r, N - 1);
    b_nib_off[i] = (int64_t)gr * rowq + ((phys ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < C::kAScLoads; ++i) {
    const int slot = (wave * C::kAScLoads + i) * 64 + lane;     // 4-byte LDS slot
    const int gr = min(m0 + (slot >> 1), M - 1);
    a_sc_off[i] = (int64_t)gr * rows + ((slot & 1) << 2);
  }
#pragma unroll
  for (int i = 0; i < C::kBScLoads; ++i) {
    const int slot = (wave * C::kBScLoads + i) * 64 + lane;
    const int gr = min(n0 + (slot >> 1), N - 1);
    b_sc_off[i] = (int64_t)gr * rows + ((slot & 1) << 2);
  }

  auto issue = [&](int st) {
    uint8_t* base = smem + (st % kStages) * L::kBytes;
    const uint8_t* aq = a_q + (int64_t)st * kRowBytes;
    const uint8_t* bq = b_q + (int64_t)st * kRowBytes;
    const uint8_t* as = a_s + (int64_t)st * kScBytes;
    const uint8_t* bs = b_s + (int64_t)st * kScBytes;
#pragma unroll
    for (int i = 0; i < C::kANibLoads; ++i)
      __builtin_amdgcn_global_load_lds(
          (gbl_void_ptr)(aq + a_nib_off[i]),
          (lds_void_ptr)(base + L::kANib + (wave * C::kANibLoads + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::kBNibLoads; ++i)
      __builtin_amdgcn_global_load_lds(
          (gbl_void_ptr)(bq + b_nib_off[i]),
          (lds_void_ptr)(base + L::kBNib + (wave * C::kBNibLoads + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::kAScLoads; ++i)
      __builtin_amdgcn_global_load_lds(
          (gbl_void_ptr)(as + a_sc_off[i]),
          (lds_void_ptr)(base + L::kASc + (wave * C::kAScLoads + i) * 256), 4, 0, 0);
#pragma unroll
    for (int i = 0; i < C::kBScLoads; ++i)
      __builtin_amdgcn_global_load_lds(
          (gbl_void_ptr)(bs + b_sc_off[i]),
          (lds_void_ptr)(base + L::kBSc + (wave * C::kBScLoads + i) * 256), 4, 0, 0);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  // prologue: stages 0 .. kStages-2 in flight
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nstage) issue(s);

  for (int st = 0; st < nstage; ++st) {
    // this wave's loads of stage st have landed once at most the loads of the
    // younger stages in flight remain; the barrier extends that to all waves
    if (st + kStages - 2 < nstage) wait_vmcnt<(kStages - 2) * C::kLoads>();
    else wait_vmcnt<0>();
    workgroup_barrier();
    // the buffer refilled here was last read in iteration st-1, which every
    // wave has finished by the barrier above
    if (st + kStages - 1 < nstage) issue(st + kStages - 1);

    const uint8_t* base = smem + (st % kStages) * L::kBytes;
    Frag fa[FM], fb[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
      fa[f] = read_frag(base + L::kANib, base + L::kASc, wm * C::TM + f * 32 + li, lg);
#pragma unroll
    for (int f = 0; f < FN; ++f)
      fb[f] = read_frag(base + L::kBNib, base + L::kBSc, wn * C::TN + f * 32 + li, lg);

    auto step = [&](auto tc) {
      constexpr int T = decltype(tc)::value;
      f16x8 av[FM], bv[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) av[f] = frag_step<T>(fa[f]);
#pragma unroll
      for (int f = 0; f < FN; ++f) bv[f] = frag_step<T>(fb[f]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
  }

  // ---- epilogue: y = fl32(ga * gb) * acc.  acc[i][j] reg r holds row
  // 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of its 32x32 tile.
  const float alpha = a_g[0] * b_g[0];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * C::TN + j * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * C::TM + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (row < M && col < N)
          store_out(y, (int64_t)row * ld_y + col, acc[i][j][r] * alpha, y_dtype);
      }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_cfg(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                      void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
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
  kern<<<(unsigned)tiles, C::kThreads, smem, stream>>>((int)M, (int)N, (int)K, a.q, a.s, a.g,
                                                        b.q, b.s, b.g, y, y_dtype, ld_y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                            void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
  if (M >= 256 && N >= 256)
    return launch_cfg<256, 256, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream);
  return launch_cfg<128, 128, 2, 2>(M, N, K, a, b, y, y_dtype, ld_y, stream);
}

}  // namespace nvfp4
