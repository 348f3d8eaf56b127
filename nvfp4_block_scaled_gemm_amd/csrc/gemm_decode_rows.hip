// Weight-streaming NVFP4 GEMM for up to 16 tokens that reads the weights in
// whole rows, in an order that keeps the chip's concurrent reads in one
// compact address window.
//
// Decode-sized GEMMs sit far below the compute ridge (magik.net "The Moment of
// Recalibration", "Input Knowledge": 16-64 token batches reach a small
// fraction of the big-GEMM rate; "The Moment of Synthesis", "The Reasoning
// Process": ~72x below the ridge), so the kernel's time is the time HBM takes
// to deliver the packed weights once.  Measured on the MI355X, a 38 MB weight
// read is fastest when every workgroup fetches whole contiguous rows and all
// workgroups work inside one window at a time (chunk c of workgroup g is rows
// R (G c + g) .. R (G c + g) + R - 1, G workgroups), with 2-3 chunks in
// flight per CU; tile-shaped chunks (32 rows x 512 bytes) or deeper rings
// stream slower.
//
// Layout of the products.  A chunk is R rows x all of K.  The MFMA
// (v_mfma_f32_16x16x32_f16, A = 16 rows, B = 16 columns) takes 16 "virtual
// rows": row r of the chunk cut into P = 16 / R parts of K / P elements,
// virtual row v = R p + r.  B's 16 columns are (part p', token t) pairs,
// column R p' + t, so one MFMA carries R token slots; the products whose
// parts agree (p == p') are the ones kept, and the parts and waves are summed
// afterwards.  NB MFMAs per step cover up to NB R tokens.
//  * The tokens' operand never changes from chunk to chunk (every chunk spans
//    all of K), so each wave dequantises its slice of x to fp16 once, into
//    registers, and each chunk dequantises only the weights: one conversion
//    and one packed multiply per pair of weight elements, the minimum for
//    exact E2M1 x E4M3 products on fp16 MFMA.
//  * Waves split each part's K range: wave w owns elements
//    [p K/P + w K/(8P), + K/(8P)) of every virtual row, lane (li, lq) the
//    8 S contiguous elements starting 8 S lq inside that (S steps per chunk).
//  * Chunks arrive by 16-byte buffer-to-LDS loads, 1 KB per instruction,
//    into a D-slot ring (D - 1 chunks in flight), one barrier per chunk.
//    The 16-byte granules of each 1 KB block are XOR-swizzled by the block's
//    virtual row, so the 16 virtual rows of a fragment read conflict-free.
//  * The barrier per chunk puts each chunk's compute latency on the critical
//    path, so a chunk does as little as possible: its LDS reads are issued
//    together, its steps alternate between two accumulators (half the
//    dependent MFMA chain), and its partial sums are only parked: each wave
//    stores the lanes that hold kept products (1 / P of them) to a compact
//    per-chunk area in LDS.  After the last chunk all threads sum every
//    chunk's partials (a fixed pairwise order over waves and parts), scale
//    by fl32(ga gb) and store fp32 or bf16.
#include "nvfp4_device.h"
#include "nvfp4_dispatch.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr uint32_t kOob = 0xFFFFFFF0u;  // past every operand: reads zero, no traffic

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(const void* p, uint32_t bytes, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(p, bytes), (lds_void_ptr)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

// Barrier that is also a compiler memory barrier, without the drain of every
// memory counter __syncthreads() implies (loads in flight target other slots).
__device__ __forceinline__ void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Compile-time shape of one configuration: R rows per chunk, K = 1024 KS,
// NB token groups of R tokens, D ring slots, W waves per workgroup.
template <int R, int KS, int NB, int D, int W>
struct Cfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int P = 16 / R;                 // parts per row (virtual rows = 16)
  static constexpr int K = 1024 * KS;
  static constexpr int S = K / (W * P * 32);       // MFMA steps per wave per chunk
  static constexpr int kNib = R * K / 2;           // nibble bytes per chunk
  static constexpr int kSc = R * K / 16;           // scale bytes per chunk
  static constexpr int kSlot = kNib + kSc;
  static constexpr int kDmaNib = kNib / 1024, kDmaSc = kSc / 1024, kDma = kDmaNib + kDmaSc;
  static constexpr int kPerWave = (kDma + kWaves - 1) / kWaves;
  static constexpr int kRowBytes = K / 2;          // one row's nibbles
  static constexpr int kPartBytes = kRowBytes / P; // one virtual row's nibbles
  static constexpr bool kPadding = kDma % W != 0;
  static constexpr int kPad = D * kSlot;                        // 1 KB sink for padding loads
  static constexpr int kPart = kPad + (kPadding ? 1024 : 0);    // parked partials
  static constexpr int kPartChunk = NB * kWaves * (4 * R) * 16; // bytes of one chunk's partials
  static constexpr int kLdsMax = 160 * 1024;
  static_assert(R == 4 || R == 8 || R == 16, "rows per chunk");
  static_assert(kPartBytes % 1024 == 0, "every 1 KB block belongs to one virtual row");
  static_assert(kSc % 1024 == 0, "whole 1 KB scale blocks");
  static_assert(S % 8 == 0, "a lane's nibbles and scales come in whole 16- and 4-byte pieces");
  static_assert(kPart + kPartChunk <= kLdsMax, "LDS budget");
  static_assert(NB * S * 4 <= 128, "register budget of the tokens' fp16 operand");
};

template <int R, int KS, int NB, int D, int W>
__global__ __launch_bounds__(64 * W, 1) void decode_rows_kernel(
    int N, int M, const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
    const float* __restrict__ a_g, const uint8_t* __restrict__ b_q,
    const uint8_t* __restrict__ b_s, const float* __restrict__ b_g, void* __restrict__ y,
    int y_dtype, int64_t ld_y) {
  using C = Cfg<R, KS, NB, D, W>;
  constexpr int P = C::P, S = C::S, K = C::K, kWaves = W, kThreads = 64 * W;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  // parked partials [chunk][nb][wave][4R kept lanes][4]
  float* const part = reinterpret_cast<float*>(smem + C::kPart);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int G = (int)gridDim.x, g = (int)blockIdx.x;
  const int groups = (N + R - 1) / R;
  const int nchunks = g < groups ? (groups - g + G - 1) / G : 0;  // uniform
  constexpr uint32_t qrow = K / 2, srow = K / 16;
  const uint32_t wq_bytes = (uint32_t)N * qrow, ws_bytes = (uint32_t)N * srow;
  const float alpha = a_g[0] * b_g[0];  // read early: off the end of the kernel
  const uint32_t inv_m = (65535u + (uint32_t)M) / (uint32_t)M;  // ceil(65536 / M)

  // ---- the tokens' operand: B column li = (part li / R, token slot
  // li % R) of token group nb; lane (li, lq) holds the 8 S elements starting
  // at p' K/P + w K/(8P) + 8 S lq.  Loaded before the first weight chunks go
  // out, dequantised to fp16 once (into registers) while they are in flight.
  u32x4 xq[NB][S / 4];
  uint32_t xs[NB][S / 8];
  {
    const auto rq = rsrc(a_q, (uint32_t)M * qrow), rs = rsrc(a_s, (uint32_t)M * srow);
    const uint32_t e0 = (uint32_t)((li / R) * (K / P) + wave * (K / (kWaves * P)) + 8 * S * lq);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = nb * R + li % R;
      const bool in = t < M;
#pragma unroll
      for (int j = 0; j < S / 4; ++j)
        xq[nb][j] = ld16(rq, in ? (uint32_t)t * qrow + e0 / 2 + 16u * j : kOob);
#pragma unroll
      for (int j = 0; j < S / 8; ++j) xs[nb][j] = ld4(rs, in ? (uint32_t)t * srow + e0 / 16 + 4u * j : kOob);
    }
  }

  // ---- this wave's DMA instructions of a chunk (instruction i -> wave i % 8).
  // Nibble block i holds virtual row v(i) and the granule at DMA position pos
  // is global granule pos ^ (v & 15); scale blocks are copied as they are.
  uint32_t voff0[C::kPerWave];   // byte offset inside a chunk (kOob: padding)
  uint32_t rowof[C::kPerWave];   // chunk-relative row the block lies in
  int ldsoff[C::kPerWave];
  bool isnib[C::kPerWave];
#pragma unroll
  for (int k = 0; k < C::kPerWave; ++k) {
    const int i = wave + kWaves * k;
    voff0[k] = kOob;
    rowof[k] = 0;
    ldsoff[k] = -1;                    // padding: the 1 KB sink, never read
    isnib[k] = true;
    if (i < C::kDmaNib) {
      const int r = (1024 * i) / C::kRowBytes;
      const int p = ((1024 * i) % C::kRowBytes) / C::kPartBytes;
      const int v = R * p + r;
      voff0[k] = 1024u * i + 16u * (uint32_t)(lane ^ (v & 15));
      rowof[k] = r;
      ldsoff[k] = 1024 * i;
    } else if (i < C::kDma) {
      const int i2 = i - C::kDmaNib;
      voff0[k] = 1024u * i2 + 16u * lane;
      rowof[k] = (1024 * i2 + 16 * lane) / srow;
      ldsoff[k] = C::kNib + 1024 * i2;
      isnib[k] = false;
    }
  }

  // Every wave issues exactly kPerWave loads per chunk (chunks past the end
  // and padding read nothing), so one fixed vmcnt wait per chunk suffices.
  auto issue = [&](int c, int slot) {
    const bool live = G * c + g < groups;  // c < nchunks, without the division
    const uint32_t row0 = (uint32_t)(R * (G * c + g));
#pragma unroll
    for (int k = 0; k < C::kPerWave; ++k) {
      const bool ok = live && voff0[k] != kOob && row0 + rowof[k] < (uint32_t)N;
      uint8_t* dst = ldsoff[k] < 0 ? smem + C::kPad : smem + slot * C::kSlot + ldsoff[k];
      if (isnib[k]) dma16(b_q, wq_bytes, ok ? row0 * qrow + voff0[k] : kOob, dst);
      else dma16(b_s, ws_bytes, ok ? row0 * srow + voff0[k] : kOob, dst);
    }
  };

  // Lane (li, lq) reads virtual row v = li: part p = li / R, row r = li % R.
  const int pv = li / R, rv = li % R;
  const uint32_t ebase = (uint32_t)(pv * (K / P) + wave * (K / (kWaves * P)) + 8 * S * lq);
  const uint32_t nib_base = (uint32_t)(rv * C::kRowBytes) + ebase / 2;   // byte in the chunk
  const uint32_t sc_base = (uint32_t)C::kNib + (uint32_t)(rv * srow) + ebase / 16;

  // Lane (li, lq) keeps its products when its column's part li / R equals
  // its rows' part (4 lq) / R; such a lane holds rows 4 (lq % (R/4)) + i,
  // i < 4, of part li / R, token slot li % R, and parks them at kept-lane
  // index li (R/4) + lq % (R/4).
  const bool kept = li / R == (4 * lq) / R;
  const int kidx = li * (R / 4) + lq % (R / 4);

#pragma unroll
  for (int c = 0; c < D - 1; ++c) issue(c, c);

  // step s = 8j + T: dword s of the nibbles (elements 8s .. 8s+7), block
  // s / 2, i.e. byte T / 2 of scale word j
  f16x8 xb[NB][S];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < S / 8; ++j) {
      const Scales sx = to_scales(xs[nb][j]);
      static_for<8>([&](auto tc) {
        constexpr int T = decltype(tc)::value;
        xb[nb][8 * j + T] = dequant_step<T>(xq[nb][(8 * j + T) / 4][T % 4], sx);
      });
    }
  int slot = 0;
  for (int c = 0; c < nchunks; ++c) {
    wait_vmcnt<(D - 2) * C::kPerWave>();
    workgroup_barrier();
    issue(c + D - 1, slot == 0 ? D - 1 : slot - 1);
    const uint8_t* sl = smem + slot * C::kSlot;
    uint32_t sw4[S / 8];
#pragma unroll
    for (int j = 0; j < S / 8; ++j)
      sw4[j] = *reinterpret_cast<const uint32_t*>(sl + sc_base + 4 * j);
    u32x4 w4[S / 4];
#pragma unroll
    for (int gq = 0; gq < S / 4; ++gq) {
      // granule gq of the lane's nibbles, swizzled inside its 1 KB block
      const uint32_t b = nib_base + 16u * gq;
      const uint32_t pos = (b & ~1023u) | ((((b >> 4) & 63u) ^ (uint32_t)li) << 4);
      w4[gq] = *reinterpret_cast<const u32x4*>(sl + pos);
    }
    f32x4 acc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb][0] = acc[nb][1] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int gq = 0; gq < S / 4; ++gq) {
      const Scales sw = to_scales(sw4[gq / 2]);
      static_for<4>([&](auto tc) {
        constexpr int T4 = decltype(tc)::value;
        // step 4 gq + T4: dword T4 of the granule, block (4 gq + T4) / 2 =
        // scale byte 2 (gq % 2) + T4 / 2 of the word
        f16x8 a;
        if (gq % 2 == 0) a = dequant_step<T4>(w4[gq][T4], sw);
        else a = dequant_step<T4 + 4>(w4[gq][T4], sw);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][T4 & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, xb[nb][4 * gq + T4],
                                                                   acc[nb][T4 & 1], 0, 0, 0);
      });
    }
    if (kept) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<f32x4*>(part + (((c * NB + nb) * kWaves + wave) * (4 * R) + kidx) * 4) =
            acc[nb][0] + acc[nb][1];
    }
    slot = slot == D - 1 ? 0 : slot + 1;
  }
  wait_vmcnt<0>();
  __syncthreads();
  // every chunk's outputs: token t, row r of chunk c, summed over waves and
  // parts in a fixed pairwise order; consecutive threads write consecutive
  // output columns.  All W P partials of an output are read before the
  // first add, so the reads overlap instead of waiting one by one.
  for (int idx = tid; idx < nchunks * M * R; idx += kThreads) {
    // idx = (c M + t) R + r; c by a multiply and a shift, exact while
    // c M + t < 65536 / M (the LDS holds far fewer chunks' partials)
    const int ct = idx / R, r = idx % R;
    const int c = (int)(((uint32_t)ct * inv_m) >> 16), t = ct - c * M;
    const int nb = t / R, tt = t % R;
    static_assert((kWaves * P & (kWaves * P - 1)) == 0, "pairwise sum over a power of two");
    float v[kWaves * P];
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int k = (R * p + tt) * (R / 4) + (r >> 2);
        v[w * P + p] = part[(((c * NB + nb) * kWaves + w) * (4 * R) + k) * 4 + (r & 3)];
      }
#pragma unroll
    for (int h = kWaves * P / 2; h >= 1; h /= 2)
#pragma unroll
      for (int i = 0; i < h; ++i) v[i] += v[i + h];
    const int n = R * (G * c + g) + r;
    if (n < N) store_out(y, (int64_t)t * ld_y + n, v[0] * alpha, y_dtype);
  }
}

int compute_units() {
  static int num_cu = 0;  // of the current device, one query per process
  if (num_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    num_cu = n;
  }
  return num_cu;
}

// Returns false (nothing launched) when the parked partials of the largest
// workgroup would not fit the LDS; *err holds the launch status otherwise.
template <int R, int KS, int NB, int D, int W>
bool launch(int64_t M, int64_t N, PackedOperand a, PackedOperand b, void* y, int y_dtype,
            int64_t ld_y, hipStream_t stream, hipError_t* err) {
  using C = Cfg<R, KS, NB, D, W>;
  auto kern = decode_rows_kernel<R, KS, NB, D, W>;
  const int64_t groups = (N + R - 1) / R;
  const int num_cu = compute_units();
  const int grid = (int)(groups < num_cu ? groups : num_cu);
  const int64_t chunks = (groups + grid - 1) / grid;
  const int64_t lds = C::kPart + chunks * C::kPartChunk;
  if (lds > C::kLdsMax) return false;
  // once per process (thread-safe static initialisation)
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsMax);
  if (attr != hipSuccess) {
    *err = attr;
    return true;
  }
  kern<<<grid, C::kThreads, (size_t)lds, stream>>>((int)N, (int)M, a.q, a.s, a.g, b.q, b.s, b.g, y,
                                                y_dtype, ld_y);
  *err = hipGetLastError();
  return true;
}

}  // namespace

hipError_t launch_gemm_decode_rows(int64_t M, int64_t N, int64_t K, PackedOperand a,
                                   PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                                   hipStream_t stream) {
  if (!decode_rows_shape(M, K) || (y_dtype != 0 && y_dtype != 1)) return hipErrorInvalidValue;
  // Measured on the MI355X at N = K = 8192 (cache-cold W, back to back):
  // 4-row chunks with a 3-slot ring take M = 1 in ~9.3 us (a 4-slot ring:
  // ~9.9 us) against ~10.8 us for the LDS-tile kernel.  From 5 tokens on
  // the products cost more than the tile kernel's (8-row chunks keep only
  // half of each MFMA, 16-row chunks fit only a 2-slot ring), so those
  // shapes go there.
  hipError_t err = hipSuccess;
  const bool done = launch<4, 8, 1, 3, 8>(M, N, a, b, y, y_dtype, ld_y, stream, &err);
  // very wide outputs: the LDS-ring tile kernel (same operand requirements)
  if (!done) return launch_gemm_decode_lds(M, N, K, a, b, y, y_dtype, ld_y, stream);
  return err;
}

}  // namespace nvfp4
