// NVFP4 quantiser: x (fp32 | bf16) [rows, cols] -> packed E2M1 nibbles,
// E4M3FN block scales (one per 16 elements) and an fp32 global scale.
//
// Format: kernelindex "NVFP4 linear layer" (description: FP4 values with FP8
// E4M3FN scales per 16 elements); magik.net "The 3.7 PFLOPS Revelation",
// "Input Knowledge" item 2 (two values per byte, K//2 data, K//16 scales).
// Quantisation runs ahead of the GEMM and is timed apart (leverageai
// "blackwell-nvfp4-gemm-optimization", "What is this?").
//
// Semantics (the pages leave them open; the reading taken is that every
// stored quantity is rounded once from its exact real value):
//   g      = fl32(amax_t / 2688)
//   s_b    = nearest E4M3 (ties to even code, saturating at 448) to amax_b/(6g)
//   code_i = nearest E2M1 magnitude (ties to even, saturating at 6) to
//            |x_i| / (E4M3(s_b) * g); 0 when s_b == 0
//   nibble = signbit(x_i) << 3 | code_i
// All decisions are exact comparisons of the input against products of a
// few-bit midpoint and g, which are exact in fp64 (at most 31 significant
// bits), or against their fp32 neighbours chosen to give the same answer.
//
// Two kernels: an amax pass writing one partial maximum per workgroup, and an
// encode pass in which every workgroup reduces the partials (deterministic,
// no atomics, no memset), derives g, and encodes its 16-element blocks.  The
// scale code and the element codes come from gfx950's E4M3 and E2M1
// encoders (round to nearest, ties to even; checked against exact rounding
// on every midpoint and its neighbours) applied to both ends of a narrow
// interval around the quotient; where the ends disagree a midpoint lies in
// the interval and an exact test settles the code (an fp64 midpoint search
// for the scale, an fma residual sign for an element).  Tensors with
// g < 2^-88 or g >= 2^116 take exact fp64 threshold comparisons throughout.
#include "nvfp4_device.h"
#include "nvfp4_encode.h"
#include "nvfp4_internal.h"

#include <mutex>

namespace nvfp4 {
namespace {

using namespace enc;

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* lds) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = max(r, lds[w]);
  __syncthreads();
  return r;
}

// ---- amax pass ------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void amax_kernel(const void* __restrict__ x, int dtype,
                                                        int64_t rows, int64_t nblk_row,
                                                        int64_t ld_x, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t total = rows * nblk_row;
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * kThreads) {
    const int64_t r = c / nblk_row, j = c - r * nblk_row;
    Block16 b;
    load_block(x, dtype, r * ld_x + j * 16, b);
    m = max(m, block_amax_bits(b));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// ---- encode pass ----------------------------------------------------------

// Walks blocks c = first + i * stride as (row, block-in-row) without
// dividing in the loop.  With kDepth > 0 each lane keeps kDepth blocks of
// loads in flight (block i is loaded while block i - kDepth is encoded); the
// default 0 loads each block when it is encoded and relies on occupancy
// (64 registers, 8 waves per SIMD) to hide latency, which measured fastest.
#ifndef NVFP4_QUANT_DEPTH
#define NVFP4_QUANT_DEPTH 0
#endif
constexpr int kDepth = NVFP4_QUANT_DEPTH;

template <int DT, int kMode>
__device__ __forceinline__ void encode_all(const void* __restrict__ x, int64_t rows,
                                           int64_t nblk_row, int64_t ld_x, uint8_t* __restrict__ q,
                                           uint8_t* __restrict__ s, const EncodeParams& P) {
  const int64_t total = rows * nblk_row;
  const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if (first >= total) return;
  const int64_t dr = stride / nblk_row, dj = stride - dr * nblk_row;
  auto step = [&](int64_t& rr, int64_t& jj) {
    rr += dr;
    jj += dj;
    if (jj >= nblk_row) { jj -= nblk_row; ++rr; }
  };
  int64_t r = first / nblk_row, j = first - r * nblk_row;   // block being encoded
  if constexpr (kDepth == 0) {
    for (int64_t c = first; c < total; c += stride) {
      encode_block<kMode>(unpack<DT>(load_raw<DT>(x, r * ld_x + j * 16)), P,
                          q + r * (nblk_row * 8) + j * 8, s + r * nblk_row + j);
      step(r, j);
    }
    return;
  }
  int64_t rp = r, jp = j;                                   // next block to load
  int64_t cp = first;
  RawBlock<DT> buf[kDepth > 0 ? kDepth : 1];
  static_for<kDepth>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    if (cp < total) buf[d] = load_raw<DT>(x, rp * ld_x + jp * 16);
    cp += stride;
    step(rp, jp);
  });
  for (int64_t c = first;; c += kDepth * stride) {
    bool done = false;
    static_for<kDepth>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (done) return;
      if (c + d * stride >= total) { done = true; return; }
      const Block16 b = unpack<DT>(buf[d]);
      if (cp < total) buf[d] = load_raw<DT>(x, rp * ld_x + jp * 16);
      cp += stride;
      step(rp, jp);
      encode_block<kMode>(b, P, q + r * (nblk_row * 8) + j * 8, s + r * nblk_row + j);
      step(r, j);
    });
    if (done) break;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void encode_kernel(
    const void* __restrict__ x, int64_t rows, int64_t nblk_row, int64_t ld_x,
    uint8_t* __restrict__ q, uint8_t* __restrict__ s, float* __restrict__ gscale,
    const uint32_t* __restrict__ partial, int npartial, int scale_given) {
  __shared__ uint32_t red[kThreads / 64];
  float g;
  if (scale_given) {
    g = *gscale;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
    m = block_max(m, red);
    // fl32(amax / 2688): the fp64 quotient rounds to the same fp32 as the
    // exact one, since amax / 2688 can come no closer to an fp32 rounding
    // boundary than 2^-25 / 21 relative unless it lies on it exactly.
    g = (float)((double)__uint_as_float(m) / 2688.0);
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = g;
  }
  // g is the same in every lane: make it explicitly scalar so the mode
  // branch below is uniform
  g = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(g)));
  const EncodeParams P = make_params(g);
  const int mode = encode_mode(g);
  if (mode == 0) encode_all<DT, 0>(x, rows, nblk_row, ld_x, q, s, P);
  else if (mode == 1) encode_all<DT, 1>(x, rows, nblk_row, ld_x, q, s, P);
  else encode_all<DT, 2>(x, rows, nblk_row, ld_x, q, s, P);
}

constexpr int kMaxPartials = 1024;  // the amax pass never runs more workgroups

int amax_grid(int64_t nblocks) {
  int64_t g = (nblocks + kThreads - 1) / kThreads;
  if (g > kMaxPartials) g = kMaxPartials;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

// Workspace of nvfp4_quantize_noalloc: the amax pass's partial maxima, one
// copy per GPU the library runs on, held until the process ends.  Every
// call on a GPU shares it, so calls that overlap on one GPU race.  Nothing
// in it needs clearing: each call writes every partial its encode pass
// reads.  Host code must not pass the array's name to a kernel (on the host
// it is only a stand-in); quantize_scratch() hands out its device address.
static __device__ __align__(256) uint32_t scratch[kMaxPartials];

size_t quantize_scratch_bytes() { return sizeof(scratch); }

hipError_t quantize_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with that device current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return sizeof(uint32_t) * (size_t)amax_grid(rows * (cols / 16));
}

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* q, uint8_t* s, float* gscale, bool scale_given,
                           void* workspace, hipStream_t stream) {
  const int64_t nblk_row = cols / 16;
  const int64_t nblocks = rows * nblk_row;
  const int np = amax_grid(nblocks);
  if (!scale_given) {
    amax_kernel<<<np, kThreads, 0, stream>>>(x, dtype, rows, nblk_row, ld_x,
                                             reinterpret_cast<uint32_t*>(workspace));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Encode grid: one resident round of workgroups (compute units x the
  // workgroups per CU the kernel's registers allow), so every lane walks
  // about the same number of blocks and no partial second round trails.
  static int resident[2] = {0, 0};
  int& res = resident[dtype == 1 ? 1 : 0];
  if (res == 0) {
    int dev = 0, ncu = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &per_cu, reinterpret_cast<const void*>(encode_kernel<1>), kThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &per_cu, reinterpret_cast<const void*>(encode_kernel<0>), kThreads, 0);
    res = (e == hipSuccess && ncu > 0 && per_cu > 0) ? ncu * per_cu : 2048;
  }
  int64_t eg = (nblocks + kThreads - 1) / kThreads;
  if (eg > res) eg = res;
  const uint32_t* partial = reinterpret_cast<const uint32_t*>(workspace);
  if (dtype == 1)
    encode_kernel<1><<<(int)eg, kThreads, 0, stream>>>(x, rows, nblk_row, ld_x, q, s, gscale,
                                                        partial, np, scale_given ? 1 : 0);
  else
    encode_kernel<0><<<(int)eg, kThreads, 0, stream>>>(x, rows, nblk_row, ld_x, q, s, gscale,
                                                        partial, np, scale_given ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4
