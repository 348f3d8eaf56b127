// NVFP4 GEMM for large M on the gfx950 matrix cores.
//
// y[m, n] = fl32(ga * gb) * sum_k A(m, k) B(n, k), A = x [M, K], B = W [N, K]
// (kernelindex "NVFP4 linear layer", description).  The pages' own kernels
// (CUTLASS / Colfax on SM120, magik.net "The Moment of Synthesis", "The
// Context That Led Here") consume FP4 natively with 128x128 tiles limited by
// 99 KB of shared memory; here the design follows CDNA4 instead:
//
//  * Packed nibbles and scale bytes (0.5625 B per element) stream from HBM
//    with 16-byte loads into a double-buffered LDS ring, one 128-deep K stage
//    at a time (64 nibble bytes + 8 scale bytes per row).
//  * Each wave reads its fragments from LDS still packed, dequantises them in
//    registers to fp16 (exact: E2M1 * E4M3 has <= 6 significant bits), and
//    issues v_mfma_f32_16x16x32_f16 with fp32 accumulation.  The E4M3 scale is
//    applied exactly by one packed fp16 multiply per element pair, so the
//    16-element blocks never need a per-block correction of the accumulator.
//  * K is permuted inside a stage, identically for A and B (a contraction is
//    order-free): lane group q = lane / 16 owns stage elements [32q, 32q+32),
//    and MFMA step j takes its dword j, so one b128 LDS read feeds four MFMAs.
//  * Workgroup tiles are mapped XCD-aware: consecutive hardware workgroup ids
//    land on different XCDs, so ids are regrouped so that each XCD works on a
//    compact block of output tiles and shares A/B rows in its own L2.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kBK = 128;        // K elements per stage
constexpr int kRowBytes = 64;   // nibble bytes per row per stage
constexpr int kRowStride = 80;  // LDS row stride: 16-byte pad, conflict-free b128 reads
constexpr int kScBytes = 8;     // scale bytes per row per stage

template <int BM, int BN>
struct Smem {
  static constexpr int kANib = 0;
  static constexpr int kASc = kANib + BM * kRowStride;
  static constexpr int kBNib = kASc + BM * kScBytes;
  static constexpr int kBSc = kBNib + BN * kRowStride;
  static constexpr int kBytes = kBSc + BN * kScBytes;  // one stage
};

// {S, S} as fp16 bits with S = E4M3(byte) * 2^-8: E4M3 and fp16 share the
// subnormal/normal structure, so the 7 magnitude bits shifted left by 7 are
// exactly E4M3 * 2^-8 in fp16 (possibly subnormal); the sign moves to bit 15.
// The factor 2^8 is restored by converting nibbles with a scale of 256.
__device__ __forceinline__ uint32_t scale_pair_bits(uint32_t byte) {
  const uint32_t h = ((byte & 0x7Fu) << 7) | ((byte & 0x80u) << 8);
  return h | (h << 16);
}

__device__ __forceinline__ f16x8 dequant8_scaled(uint32_t packed, uint32_t pair_bits) {
  f16x2 s2;
  __builtin_memcpy(&s2, &pair_bits, 4);
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 0);
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 1);
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 2);
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 256.0f, 3);
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Regroup hardware workgroup ids so that each of the 8 XCDs (which receive
// ids round-robin) owns a contiguous range of logical tiles, then walk that
// range in column groups of GROUP_M tile-rows for L2 reuse.
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

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(256, 1) void gemm_mfma_kernel(
    int M, int N, int K, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y) {
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_CHUNKS = BM * 4 / 256, B_CHUNKS = BN * 4 / 256;  // 16-byte chunks / thread
  using L = Smem<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int li = lane & 15, lq = lane >> 4;

  int tm, tn;
  tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowq = K / 2, rows = K / 16;  // bytes per operand row
  const int nstage = K / kBK;

  // ---- global -> register prefetch of one stage ----
  u32x4 pa[A_CHUNKS], pb[B_CHUNKS];
  u32x2 psa = {0, 0}, psb = {0, 0};
  auto fetch = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + 256 * i, r = c >> 2, part = c & 3;
      const int gr = m0 + r;
      pa[i] = (gr < M) ? *reinterpret_cast<const u32x4*>(a_q + gr * rowq + st * kRowBytes + part * 16)
                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int c = tid + 256 * i, r = c >> 2, part = c & 3;
      const int gr = n0 + r;
      pb[i] = (gr < N) ? *reinterpret_cast<const u32x4*>(b_q + gr * rowq + st * kRowBytes + part * 16)
                       : u32x4{0, 0, 0, 0};
    }
    if (tid < BM) {
      const int gr = m0 + tid;
      psa = (gr < M) ? *reinterpret_cast<const u32x2*>(a_s + gr * rows + st * kScBytes) : u32x2{0, 0};
    }
    if (tid < BN) {
      const int gr = n0 + tid;
      psb = (gr < N) ? *reinterpret_cast<const u32x2*>(b_s + gr * rows + st * kScBytes) : u32x2{0, 0};
    }
  };
  auto stash = [&](int buf) {
    uint8_t* base = smem + buf * L::kBytes;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + 256 * i, r = c >> 2, part = c & 3;
      *reinterpret_cast<u32x4*>(base + L::kANib + r * kRowStride + part * 16) = pa[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int c = tid + 256 * i, r = c >> 2, part = c & 3;
      *reinterpret_cast<u32x4*>(base + L::kBNib + r * kRowStride + part * 16) = pb[i];
    }
    if (tid < BM) *reinterpret_cast<u32x2*>(base + L::kASc + tid * kScBytes) = psa;
    if (tid < BN) *reinterpret_cast<u32x2*>(base + L::kBSc + tid * kScBytes) = psb;
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  fetch(0);
  stash(0);
  __syncthreads();

  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstage) fetch(st + 1);
    const uint8_t* base = smem + buf * L::kBytes;

    u32x4 ak[FM], bk[FN];
    uint32_t as2[FM], bs2[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = wm * TM + f * 16 + li;
      ak[f] = *reinterpret_cast<const u32x4*>(base + L::kANib + r * kRowStride + lq * 16);
      as2[f] = *reinterpret_cast<const uint16_t*>(base + L::kASc + r * kScBytes + lq * 2);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int r = wn * TN + f * 16 + li;
      bk[f] = *reinterpret_cast<const u32x4*>(base + L::kBNib + r * kRowStride + lq * 16);
      bs2[f] = *reinterpret_cast<const uint16_t*>(base + L::kBSc + r * kScBytes + lq * 2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 af[FM], bf[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f)
        af[f] = dequant8_scaled(ak[f][j], scale_pair_bits((as2[f] >> (8 * (j >> 1))) & 0xFFu));
#pragma unroll
      for (int f = 0; f < FN; ++f)
        bf[f] = dequant8_scaled(bk[f][j], scale_pair_bits((bs2[f] >> (8 * (j >> 1))) & 0xFFu));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
    }
    if (st + 1 < nstage) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: y = fl32(ga * gb) * acc ----
  const float alpha = a_g[0] * b_g[0];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = n0 + wn * TN + fn * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * TM + fm * 16 + lq * 4 + r;
        if (row < M && col < N) store_out(y, (int64_t)row * ld_y + col, acc[fm][fn][r] * alpha, y_dtype);
      }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_cfg(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                      void* y, int y_dtype, int64_t ld_y, hipStream_t stream) {
  using L = Smem<BM, BN>;
  const int smem = 2 * L::kBytes;
  auto kern = gemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N>;
  // once per process (thread-safe static initialisation)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  kern<<<(unsigned)tiles, 256, smem, stream>>>((int)M, (int)N, (int)K, a.q, a.s, a.g, b.q, b.s,
                                               b.g, y, y_dtype, ld_y);
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
