// Weight-streaming NVFP4 GEMM for up to 32 tokens (the decode case), with
// every operand byte brought into LDS by buffer-to-LDS DMA through a deep ring.
//
// The pages place decode-sized GEMMs far below the compute ridge (magik.net
// "The Moment of Recalibration", "Input Knowledge": 16-64 token batches reach
// a small fraction of the big-GEMM rate; "The Moment of Synthesis", "The
// Reasoning Process": the per-expert GEMMs sit ~72x below the ridge).  The
// job is to move the packed weights from HBM once, at the rate the memory
// system gives, with the exact dequantise-and-multiply work hidden under it.
// The kernel keeps a few chunks of its weight tile in flight per CU:
//
//  * One workgroup (8 waves) owns 32 weight rows (output columns) over all
//    of K; K is walked in chunks of 1024 elements.  A chunk is 32 rows x
//    512 B of weight nibbles + 32 x 64 B of weight scales + the tokens'
//    rows of the same K range (M x 512 B + M x 64 B; from L2, every
//    workgroup reads them).
//  * Every chunk goes to LDS with 16-byte buffer-to-LDS loads, 1 KB per
//    instruction, each covering whole 128-byte lines of two rows.  The ring
//    holds 3 chunks, 2 of them in flight while one is multiplied (for 5-32
//    tokens; 2 or 4 slots measured slower, deeper rings slower still).
//    One barrier per chunk separates the landing of chunk c from the reuse
//    of the slot that held chunk c - 1.
//  * Inside a chunk wave w takes K elements [128w, 128w + 128): lane (li, lq)
//    holds 32 contiguous elements (16 bytes, two 16-element blocks) of row
//    li of each 16-row fragment, for four v_mfma_f32_16x16x32_f16 steps with
//    the weights as the A operand and the tokens as B.  K is permuted the
//    same way on both sides.  Both operands are dequantised exactly to fp16
//    in registers (every E2M1 x E4M3 product is an fp16 number).
//  * Rows are stored in LDS with their 16-byte chunks XOR-swizzled by the
//    row index (chunk j of row r at position j ^ (r % 16)), so the 16 rows of
//    a fragment read conflict-free; the swizzle is applied by choosing which
//    global chunk each DMA lane fetches, so the loads still cover whole lines.
//  * Token rows at or beyond M read from a 1 KB area of zeros, never from
//    the ring, so nothing depends on what out-of-range loads leave in LDS.
//  * The 8 waves' partial tiles are summed through LDS in a fixed order
//    (deterministic, no atomics), scaled by fl32(ga * gb) and stored as fp32,
//    bf16 (round to nearest even) or NVFP4 (exact block encoder).
#include "nvfp4_device.h"
#include "nvfp4_encode.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;                  // weight rows per workgroup
constexpr int kChunkK = 1024;              // K elements per chunk
constexpr int kRowNib = kChunkK / 2;       // 512 nibble bytes per row per chunk
constexpr int kRowSc = kChunkK / 16;       // 64 scale bytes per row per chunk
constexpr uint32_t kOob = 0xFFFFFFF0u;     // past every operand: reads zero, no traffic

// LDS layout of one ring slot for MX reserved token rows (every region is
// whole 1 KB DMA destinations).
template <int MX>
struct Slot {
  static constexpr int kWNib = 0;
  static constexpr int kWSc = kWNib + kRows * kRowNib;           // 16 KB
  static constexpr int kXNib = kWSc + kRows * kRowSc;            // + 2 KB
  static constexpr int kXSc = kXNib + MX * kRowNib;
  static constexpr int kBytes = kXSc + ((MX + 15) / 16) * 1024;
  // DMA instructions per chunk: weight nibbles (2 rows each), weight scales
  // (16 rows each), token nibbles, token scales
  static constexpr int kDmaW = kRows * kRowNib / 1024;
  static constexpr int kDmaWs = kRows * kRowSc / 1024;
  static constexpr int kDmaX = MX * kRowNib / 1024;
  static constexpr int kDmaXs = (MX + 15) / 16;
  static constexpr int kDma = kDmaW + kDmaWs + kDmaX + kDmaXs;
  static constexpr int kPerWave = (kDma + kWaves - 1) / kWaves;  // padded to equal counts
  static_assert(MX % 2 == 0, "token rows come in pairs per DMA");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(const void* p, uint32_t bytes, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(p, bytes), (lds_void_ptr)lds, 16, voff, 0, 0, 0);
}

// Workgroup barrier that is also a compiler memory barrier, without the
// drain of every memory counter that __syncthreads() implies: the loads
// still in flight target other ring slots, and each wave has already waited
// for its own loads of the chunk about to be read.
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One of a wave's DMA instructions per chunk: source buffer (uniform), this
// lane's byte offset in chunk 0 (kOob: nothing to fetch), the offset step
// per chunk and the LDS destination inside a slot (uniform; < 0: the zero
// area, for padding instructions).
struct Dma {
  const uint8_t* base;
  uint32_t bytes;
  uint32_t voff;
  uint32_t step;
  int lds;
};

template <int NX, int MX, int D>
__global__ __launch_bounds__(kThreads, 1) void decode_lds_kernel(
    int N, int K, int M, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y, QuantOut qo) {
  using L = Slot<MX>;
  static_assert(16 * NX >= MX, "reserved token rows fit the token fragments");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t* const zero = smem + D * L::kBytes;  // 1 KB of zeros

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int n0 = (int)blockIdx.x * kRows;
  const uint32_t qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
  const int nchunks = K / kChunkK;

  if (tid < 64) *reinterpret_cast<u32x4*>(zero + 16 * tid) = u32x4{0, 0, 0, 0};

  // This wave's DMA instructions: instruction i of a chunk belongs to wave
  // i % 8.  Nibble instructions: lane L fetches row 2i' + L/32, DMA position
  // p = L % 32 of the row's 512 bytes, holding global 16-byte chunk
  // p ^ (row % 16).  Scale instructions: row 16i' + L/4, bytes 16 (L % 4).
  Dma dma[L::kPerWave];
#pragma unroll
  for (int k = 0; k < L::kPerWave; ++k) {
    const int i = wave + kWaves * k;
    Dma d{b_q, 0u, kOob, 0u, -1};
    if (i < L::kDmaW) {
      const int r = 2 * i + (lane >> 5), p = lane & 31;
      d = Dma{b_q, (uint32_t)N * qrow,
              n0 + r < N ? (uint32_t)(n0 + r) * qrow + (uint32_t)((p ^ (r & 15)) << 4) : kOob,
              (uint32_t)kRowNib, L::kWNib + 1024 * i};
    } else if (i < L::kDmaW + L::kDmaWs) {
      const int i2 = i - L::kDmaW, r = 16 * i2 + (lane >> 2);
      d = Dma{b_s, (uint32_t)N * srow,
              n0 + r < N ? (uint32_t)(n0 + r) * srow + (uint32_t)((lane & 3) << 4) : kOob,
              (uint32_t)kRowSc, L::kWSc + 1024 * i2};
    } else if (i < L::kDmaW + L::kDmaWs + L::kDmaX) {
      const int i2 = i - L::kDmaW - L::kDmaWs, t = 2 * i2 + (lane >> 5), p = lane & 31;
      d = Dma{a_q, (uint32_t)M * qrow,
              t < M ? (uint32_t)t * qrow + (uint32_t)((p ^ (t & 15)) << 4) : kOob,
              (uint32_t)kRowNib, L::kXNib + 1024 * i2};
    } else if (i < L::kDma) {
      const int i2 = i - L::kDmaW - L::kDmaWs - L::kDmaX, t = 16 * i2 + (lane >> 2);
      d = Dma{a_s, (uint32_t)M * srow,
              t < M ? (uint32_t)t * srow + (uint32_t)((lane & 3) << 4) : kOob,
              (uint32_t)kRowSc, L::kXSc + 1024 * i2};
    }
    dma[k] = d;
  }

  // Every wave issues exactly kPerWave loads per chunk (chunks past K and
  // padding instructions read nothing), so one fixed vmcnt wait per chunk
  // suffices.
  auto issue = [&](int c, int slot) {
    const bool live = c < nchunks;
#pragma unroll
    for (int k = 0; k < L::kPerWave; ++k) {
      const uint32_t v = live && dma[k].voff != kOob ? dma[k].voff + (uint32_t)c * dma[k].step : kOob;
      dma16(dma[k].base, dma[k].bytes, v,
            dma[k].lds >= 0 ? smem + slot * L::kBytes + dma[k].lds : zero);
    }
  };

  f32x4 acc[2][NX];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < NX; ++g) acc[f][g] = f32x4{0, 0, 0, 0};

  // Lane (li, lq) of wave w reads logical 16-byte chunk j = 4w + lq of a row
  // (K elements 32j .. 32j + 31 of the chunk) and scale bytes 2j, 2j + 1.
  const int j = 4 * wave + lq;
  auto compute = [&](int slot) {
    const uint8_t* sl = smem + slot * L::kBytes;
    u32x4 wn[2];
    Scales sw[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int r = 16 * f + li;
      wn[f] = *reinterpret_cast<const u32x4*>(sl + L::kWNib + r * kRowNib + ((j ^ (r & 15)) << 4));
      sw[f] = to_scales(*reinterpret_cast<const uint16_t*>(sl + L::kWSc + r * kRowSc + 2 * j));
    }
    u32x4 xn[NX];
    Scales sx[NX];
#pragma unroll
    for (int g = 0; g < NX; ++g) {
      const int t = 16 * g + li;
      const bool in = t < M;
      const uint8_t* pn = in ? sl + L::kXNib + t * kRowNib + ((j ^ (t & 15)) << 4) : zero;
      const uint8_t* ps = in ? sl + L::kXSc + t * kRowSc + 2 * j : zero;
      xn[g] = *reinterpret_cast<const u32x4*>(pn);
      sx[g] = to_scales(*reinterpret_cast<const uint16_t*>(ps));
    }
    // step T uses dword T of the 16 bytes: elements 8T .. 8T + 7, block T / 2
    static_for<4>([&](auto tc) {
      constexpr int T = decltype(tc)::value;
      const f16x8 a0 = dequant_step<T>(wn[0][T], sw[0]);
      const f16x8 a1 = dequant_step<T>(wn[1][T], sw[1]);
#pragma unroll
      for (int g = 0; g < NX; ++g) {
        const f16x8 b = dequant_step<T>(xn[g][T], sx[g]);
        acc[0][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b, acc[0][g], 0, 0, 0);
        acc[1][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b, acc[1][g], 0, 0, 0);
      }
    });
  };

  // Ring: chunks 0 .. D-2 go out first.  Iteration c waits for its own loads
  // of chunk c (D - 2 younger chunks may stay in flight), meets the other
  // waves at the barrier (after which every wave's part of chunk c has
  // landed and every wave is done with chunk c - 1), refills chunk c - 1's
  // slot with chunk c + D - 1, then multiplies chunk c.
#pragma unroll
  for (int c = 0; c < D - 1; ++c) issue(c, c);
  int slot = 0;
  for (int c = 0; c < nchunks; ++c) {
    wait_vmcnt<(D - 2) * L::kPerWave>();
    workgroup_barrier();
    issue(c + D - 1, slot == 0 ? D - 1 : slot - 1);
    compute(slot);
    slot = slot == D - 1 ? 0 : slot + 1;
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Fixed-order sum of the 8 partial tiles through LDS (the ring is free):
  // acc[f][g] reg r is weight row 16f + 4lq + r, token 16g + li.
  constexpr int kTok = 16 * NX, kLd = kTok + 1;
  float* red = reinterpret_cast<float*>(smem);                         // [8][32][kLd]
  float* yt = reinterpret_cast<float*>(smem + kWaves * kRows * kLd * 4); // [kTok][kRows + 4]
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int g = 0; g < NX; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(wave * kRows + 16 * f + 4 * lq + r) * kLd + 16 * g + li] = acc[f][g][r];
  __syncthreads();
  const float alpha = a_g[0] * b_g[0];
#pragma unroll
  for (int h = 0; h < kTok * kRows / kThreads; ++h) {
    const int o = tid + h * kThreads;
    const int tok = o >> 5, wr = o & 31;
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) s += red[(v * kRows + wr) * kLd + tok];
    const int n = n0 + wr;
    if (y_dtype == 2) yt[tok * (kRows + 4) + wr] = s * alpha;
    else if (tok < M && n < N) store_out(y, (int64_t)tok * ld_y + n, s * alpha, y_dtype);
  }
  if (y_dtype == 2) {  // uniform
    // the same fp32 values, quantised with the given global scale: lane t
    // of the first waves encodes token t / 2's block t % 2 (16 columns)
    __syncthreads();
    if (tid < 2 * kTok) {
      const int tok = tid >> 1, c0 = n0 + 16 * (tid & 1);
      const float g = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(qo.g[0])));
      const enc::EncodeParams P = enc::make_params(g);
      const int mode = enc::encode_mode(g);
      enc::Block16 b;
#pragma unroll
      for (int e = 0; e < 16; ++e) b.v[e] = yt[tok * (kRows + 4) + 16 * (tid & 1) + e];
      if (tok < M && c0 < N) {
        uint8_t* qp = qo.q + (int64_t)tok * (N / 2) + c0 / 2;
        uint8_t* sp = qo.s + (int64_t)tok * (N / 16) + c0 / 16;
        if (mode == 1) enc::encode_block<1>(b, P, qp, sp);
        else if (mode == 0) enc::encode_block<0>(b, P, qp, sp);
        else enc::encode_block<2>(b, P, qp, sp);
      }
    }
  }
}

template <int NX, int MX, int D>
hipError_t launch(int64_t M, int64_t N, int64_t K, PackedOperand a, PackedOperand b, void* y,
                  int y_dtype, int64_t ld_y, hipStream_t stream, QuantOut qo) {
  constexpr int smem = D * Slot<MX>::kBytes + 1024;
  static_assert(smem <= 160 * 1024, "LDS budget");
  static_assert(kWaves * kRows * (16 * NX + 1) * 4 + 16 * NX * (kRows + 4) * 4 <= D * Slot<MX>::kBytes,
                "the reduction fits in the ring");
  auto kern = decode_lds_kernel<NX, MX, D>;
  // once per process (thread-safe static initialisation)
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = (N + kRows - 1) / kRows;
  kern<<<(unsigned)tiles, kThreads, smem, stream>>>(
      (int)N, (int)K, (int)M, a.q, a.s, a.g, b.q, b.s, b.g, y, y_dtype, ld_y, qo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode_lds(int64_t M, int64_t N, int64_t K, PackedOperand a,
                                  PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                                  hipStream_t stream, QuantOut qo) {
  // Ring depth, measured on the MI355X at N = K = 8192 (cache-cold W, back
  // to back): 3 slots take M = 16 / 32 in ~10.9 / ~13.4 us against ~11.6 /
  // ~14.1 us with 4 slots and ~11.8 / ~13.6 us with 2; 5 or more slots (M =
  // 1 / 16 in ~12.7 / ~12.4 us with 7 / 5) are slower still.  Up to 4
  // tokens (K != 8192: the whole-row kernel takes K = 8192) keep 4 slots.
  if (M <= 4) return launch<1, 4, 4>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
  if (M <= 16) return launch<1, 16, 3>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
  return launch<2, 32, 3>(M, N, K, a, b, y, y_dtype, ld_y, stream, qo);
}

}  // namespace nvfp4
