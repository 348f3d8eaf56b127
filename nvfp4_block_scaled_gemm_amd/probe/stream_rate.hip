// Measurement probe (not part of the GEMM library): how fast the grouped
// GEMM's weight-load pattern can stream from HBM when nothing else runs.
// Each CU runs one workgroup of four waves, each with a private 2-slot LDS
// ring, as the grouped kernel does.  The waves walk "items" of weight rows
// with the grid stride, and each item is a sequence of 16 KB jobs.  A job's
// nibbles are 16 buffer-to-LDS loads of 1 KB, covering R rows x B bytes of
// a [rows, 3072 B] matrix (the nibbles of K = 6144).  The job's scales come
// from a [rows, 384 B] matrix in one of three patterns.  Loads run one job
// ahead; a wave then waits for the older job and, if `busy` > 0, runs a
// dependent chain of `busy` fp32 FMAs standing in for the job's products.
//
//   int probe_stream_rate(int mode, const void* w, const void* s, int n_items,
//                         int busy, int blocks, unsigned* out, void* stream)
//
// mode 0: 64-row items, jobs of 64 rows x 256 B, no scales;
// mode 1: as 0 plus scales, two loads of 32 rows x 32 B (the grouped kernel's pattern);
// mode 2: as 1 but the scales by whole 128-byte lines (8 rows per load, a line per 4 jobs);
// mode 3: 128-row items, jobs of 128 rows x 128 B, scales two loads of 64 rows x 16 B.
// w holds n_items * 64 rows of 3072 bytes and s the same rows of 384 bytes
// (both below 4 GiB).  `out` is one device word (kept live, never
// written in practice).  Returns 0, -1 for a bad mode or shape, or the HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kRowBytes = 3072, kScRow = 384, kJob = 16384, kSlot = 18432;

template <int R, int B, int IR, int SC>
__global__ __launch_bounds__(256, 1) void stream_kernel(const uint8_t* w, uint32_t bytes,
                                                        const uint8_t* sc, uint32_t sbytes,
                                                        int n_items, int busy, unsigned* out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  static_assert(IR % R == 0 && R * B == kJob, "job shape");
  constexpr int kGroups = IR / R, kRanges = kRowBytes / B, kJobsPerItem = kGroups * kRanges;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* ring = smem + wave * 2 * kSlot;
  const int stride = gridDim.x * 4;
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)bytes, 0x00020000);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)sc, (short)0, (int)sbytes, 0x00020000);

  // job jj of item it into ring slot `slot`; a finished wave reloads job 0
  auto issue = [&](int it, int jj, int slot) {
    const bool live = it < n_items;
    const int r = jj / kGroups, g = jj % kGroups;
    const uint32_t row0 = live ? (uint32_t)it * IR + (uint32_t)(g * R) : 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t e = 1024u * k + 16u * lane;  // byte of the job: row e / B, column e % B
      const uint32_t off = (row0 + e / B) * kRowBytes + (uint32_t)(r * B) + e % B;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_ptr)(ring + slot * kSlot + k * 1024), 16,
                                               off, 0, 0, 0);
    }
    if constexpr (SC == 1) {  // the job's B / 8 scale bytes of each row, 16 bytes per lane
      constexpr int PER = B / 8;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t e = 1024u * m + 16u * lane;
        const uint32_t off = (row0 + e / PER) * kScRow + (uint32_t)(r * PER) + e % PER;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(ring + slot * kSlot + kJob + m * 1024),
                                                 16, off, 0, 0, 0);
      }
    } else if constexpr (SC == 2) {  // whole lines: job jj loads 16 rows of its 4-job line
      const uint32_t line = (uint32_t)(r / 4) * 128u;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t row = row0 + 16u * (uint32_t)(jj % 4) + 8u * m + (uint32_t)(lane >> 3);
        const uint32_t off = row * kScRow + line + (uint32_t)(lane & 7) * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(ring + slot * kSlot + kJob + m * 1024),
                                                 16, off, 0, 0, 0);
      }
    }
  };

  constexpr int kLoads = SC ? 18 : 16;
  unsigned acc = 0;
  int item = blockIdx.x * 4 + wave, j = 0;
  int li = item, lj = 0, slot = 0;
  issue(li, lj, 0);
  if (++lj == kJobsPerItem) { lj = 0; li += stride; }
  while (item < n_items) {
    issue(li, lj, slot ^ 1);
    if (++lj == kJobsPerItem) { lj = 0; li += stride; }
    __builtin_amdgcn_s_waitcnt((kLoads & 15) | ((kLoads >> 4) << 14) | (7 << 4) | (15 << 8));
    acc += *reinterpret_cast<const unsigned*>(ring + slot * kSlot + lane * 16);
    if (busy > 0) {
      float f = __uint_as_float(acc & 0x3FFFFFFFu);
#pragma unroll 16
      for (int t = 0; t < busy; ++t) f = __builtin_fmaf(f, 0.999f, 1e-7f);
      acc += (unsigned)(f > 1e30f);
    }
    slot ^= 1;
    if (++j == kJobsPerItem) { j = 0; item += stride; }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the padding loads land before the wave exits
  if (acc == 0x9E3779B9u) out[0] = acc;
}

template <int R, int B, int IR, int SC>
int launch(const void* w, const void* s, int n_items, int busy, int blocks, unsigned* out,
           hipStream_t stream) {
  auto k = stream_kernel<R, B, IR, SC>;
  const int smem = 4 * 2 * kSlot;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (attr != hipSuccess) return (int)attr;
  const uint64_t rows = (uint64_t)n_items * IR;
  if (rows * kRowBytes >= (1ull << 32)) return -1;
  k<<<blocks, 256, smem, stream>>>(static_cast<const uint8_t*>(w), (uint32_t)(rows * kRowBytes),
                                    static_cast<const uint8_t*>(s), (uint32_t)(rows * kScRow),
                                    n_items, busy, out);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" int probe_stream_rate(int mode, const void* w, const void* s, int n_items, int busy,
                                 int blocks, unsigned* out, void* stream) {
  if (n_items <= 0 || blocks <= 0 || busy < 0 || w == nullptr || s == nullptr || out == nullptr)
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: return launch<64, 256, 64, 0>(w, s, n_items, busy, blocks, out, st);
    case 1: return launch<64, 256, 64, 1>(w, s, n_items, busy, blocks, out, st);
    case 2: return launch<64, 256, 64, 2>(w, s, n_items, busy, blocks, out, st);
    case 3: return launch<128, 128, 128, 1>(w, s, n_items, busy, blocks, out, st);
    default: return -1;
  }
}
