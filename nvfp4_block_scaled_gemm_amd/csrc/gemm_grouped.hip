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
//  * Work items are (expert e, 64-row weight tile); a wave owns an item over
//    all of K and all of the expert's tokens, so no partial sums ever cross
//    waves.  The waves of the grid walk the item list with a fixed stride;
//    experts without tokens are skipped.  One workgroup of four waves per CU
//    (one wave per SIMD) leaves the whole LDS to the weight rings.
//  * A wave's jobs are (item, 32-token chunk, 512-element K slice).  Lane
//    group q of a job owns the slice's K-elements [128q, 128q+128), so every
//    lane moves at least 8 contiguous bytes per load (loads of 4 bytes per
//    lane cost nearly as much memory-pipeline time as 16-byte ones).  A job
//    brings 18 KB of packed weights (64 rows x 256 B of nibbles + 32 B of
//    scales) into a private 2-slot LDS ring with 16-byte buffer-to-LDS loads,
//    and the chunk's activations (64 B of nibbles + 8 B of scales per lane
//    and token fragment) into registers.  A job issues its activation loads
//    before its weight loads, so the wait for the job ends on the weight
//    stream rather than on activations queued behind it (measured 1.5 %
//    faster on the balanced MoE shapes).  Rows past the operands read as
//    zero; token rows outside the expert's chunk are not fetched.  Loads run
//    one job ahead and every job issues the same 28 memory instructions (a
//    finished wave pads with harmless reloads), so one fixed s_waitcnt per
//    job suffices.  They go out in two parts: the activations and the first
//    four weight DMAs before the previous job's products, the other 14 DMAs
//    after its step 6 (1-2 % faster on plain grouped rows than one burst of
//    28, the same through a routing index).  Weight rows are XOR-swizzled in
//    16-byte chunks in LDS so fragment reads of 16 rows 256 B apart hit
//    distinct banks.
//  * A job dequantises both operands exactly to fp16 in registers and issues
//    v_mfma_f32_16x16x32_f16: four 16-row weight fragments x one or two
//    16-token fragments, 16 steps per job (K is permuted identically on both
//    sides).  Each token fragment is dequantised once per step and reused by
//    the four weight fragments.  The steps are software-pipelined: step T's
//    MFMAs go out beside step T+1's dequantisation, so with one wave per
//    SIMD the matrix core and the vector unit still overlap.
//  * After the last slice of an item-chunk the wave scales by ga * gb[e] and
//    stores its 64 x ntok outputs, four consecutive columns per store.
//  * One launch can carry several independent grouped GEMMs (up to
//    kMaxProblems, e.g. a mixture-of-experts layer's gate_up and down
//    projections): their items are numbered one after the other and the
//    waves walk the union, so the launch ramp, the per-CU fill and the tail
//    are shared.  A wave takes its items problem by problem, each through a
//    copy of the pipeline specialised for that problem (drained in between),
//    so the problem's sizes and operand descriptors sit in scalar registers
//    as in a single-problem launch.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

#ifndef NVFP4_GROUPED_FRAGS
#define NVFP4_GROUPED_FRAGS 4
#endif
#ifndef NVFP4_GROUPED_WAVES
#define NVFP4_GROUPED_WAVES 4
#endif
constexpr int kWaves = NVFP4_GROUPED_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kFrags = NVFP4_GROUPED_FRAGS;      // 16-row weight fragments per item
constexpr int kRows = 16 * kFrags;               // weight rows per item
constexpr int kJobK = 512;                       // K elements per job
#ifndef NVFP4_GROUPED_SLOTS
#define NVFP4_GROUPED_SLOTS 2
#endif
constexpr int kSlots = NVFP4_GROUPED_SLOTS;      // LDS ring depth per wave
constexpr int kRowNib = kJobK / 2;               // 256 B of nibbles per row per job
constexpr int kRowSc = kJobK / 16;               // 32 B of scales per row per job
constexpr int kSlotNib = kRows * kRowNib;        // nibbles of one job
constexpr int kSlotBytes = kSlotNib + kRows * kRowSc;  // + its scales
constexpr int kWaveLds = kSlots * kSlotBytes;
constexpr int kNibLoads = kRows / 4;             // 16-byte DMAs of nibbles (4 rows each)
constexpr int kScLoads = kRows / 32;             // 16-byte DMAs of scales (32 rows each)
constexpr int kLoadsPerJob = kNibLoads + kScLoads + 10;  // memory instructions per job
constexpr int kDmaA = 4;                         // weight DMAs in a job's first part
constexpr int kLoadsA = 10 + kDmaA;              // memory instructions of the first part
constexpr int kStepB = 6;                        // product step after which the second part goes
static_assert(kDmaA <= kNibLoads && kStepB < 16, "load split");
static_assert(kFrags % 2 == 0, "scale DMAs cover 32 rows");
constexpr uint32_t kOob = 0xFFFFFFF0u;           // offset past every operand (reads zero)
constexpr int kMaxProblems = kGroupedMaxProblems;
constexpr int kPrefix = 1024;                    // prefix entries per problem (LDS)
constexpr int kMaxGroups = kPrefix - 1;          // experts per problem of one launch
constexpr int kXcds = 8;                         // XCDs the workgroups go round-robin over
constexpr int kLds = kWaves * kWaveLds + kMaxProblems * kPrefix * 4;
static_assert(kLds <= 160 * 1024, "LDS budget");
static_assert(kPrefix % kThreads == 0, "experts per thread");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16(const void* p, uint32_t bytes, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(p, bytes), (lds_void_ptr)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ u32x4 ld16(const void* p, uint32_t bytes, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(p, bytes), voff, 0, 0));
}
__device__ __forceinline__ u32x2 ld8(const void* p, uint32_t bytes, uint32_t voff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsrc(p, bytes), voff, 0, 0));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One grouped GEMM of a launch (every field uniform).
struct Problem {
  const int32_t* m_offsets;  // [G + 1]
  const int32_t* row_index;  // nullptr: grouped row r reads activation row r
  const uint8_t* a_q;
  const uint8_t* a_s;
  const float* a_g;
  const uint8_t* b_q;
  const uint8_t* b_s;
  const float* b_g;
  void* y;
  int64_t ld_y;
  int64_t total_m;
  int64_t a_rows;            // rows of the activation operand
  int G, N, K, nunits, tiles;
  int y_dtype;
  uint32_t y_bytes;          // extent of y when below 4 GiB and its rows take
                             // 8-byte (bf16) / 16-byte (fp32) stores, else 0
};

struct Problems {
  Problem p[kMaxProblems];
  int count;
};

// The launch's problem list is its only argument, so it starts the
// kernel-argument segment; problem pi's fields are read from there with
// scalar loads (indexing the by-value argument instead would copy it to
// private memory).  pi is fixed across a problem's loop, so the loads are
// loop-invariant.
typedef const Problems __attribute__((address_space(4)))* ProblemsPtr;
typedef const Problem __attribute__((address_space(4)))& ProblemRef;
__device__ __forceinline__ ProblemRef problem(int pi) {
  return ((ProblemsPtr)__builtin_amdgcn_kernarg_segment_ptr())->p[pi];
}

// Read-only inputs read at uniform addresses (routing offsets and indices,
// global scales) are addressed through the constant address space, so
// they come in through the scalar cache and their wait never drains the
// vector loads in flight.  (Reached through the problem struct, the
// compiler cannot otherwise tell that the output stores leave them alone.)
template <typename T>
__device__ __forceinline__ const T __attribute__((address_space(4)))* scalar_ptr(const T* p) {
  return (const T __attribute__((address_space(4)))*)p;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Token rows [r0, r1) of expert e, clamped into [0, total_m) whatever the
// offsets hold.
template <typename Ptr>
__device__ __forceinline__ void expert_rows(Ptr m_offsets, int64_t total_m, int e, int64_t& r0,
                                            int64_t& r1) {
  int64_t a = m_offsets[e], b = m_offsets[e + 1];
  a = a < 0 ? 0 : (a > total_m ? total_m : a);
  b = b < a ? a : (b > total_m ? total_m : b);
  r0 = a;
  r1 = b;
}

// Work units.  Expert e with r_e token rows has C_e = ceil(r_e / 32)
// chunks of up to 32 tokens; a unit is (expert, 64-row weight tile,
// chunk), and a wave runs it over all of K.  Units are numbered expert by
// expert, tile by tile, chunk fastest, so expert e owns units
// [tiles * pp[e], tiles * pp[e + 1]) where pp is the prefix sum of C_e.
// Every workgroup builds pp for each problem in LDS at start (four experts
// per thread, a wave scan and a scan of the wave totals); experts without
// tokens own no units.
__device__ __forceinline__ void build_prefixes(const Problems& ps, int* pref, int* tmp) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int pi = 0; pi < ps.count; ++pi) {
    ProblemRef P = problem(pi);
    const int G = P.G;
    int* pp = pref + pi * kPrefix;
    int c[kPrefix / kThreads], sum = 0;
#pragma unroll
    for (int j = 0; j < kPrefix / kThreads; ++j) {
      const int e = (kPrefix / kThreads) * t + j;
      int n = 0;
      if (e < G) {
        int64_t r0, r1;
        expert_rows(P.m_offsets, P.total_m, e, r0, r1);
        n = (int)((r1 - r0 + 31) / 32);
      }
      sum += n;
      c[j] = sum;
    }
    int v = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(v, d, 64);
      v += lane >= d ? y : 0;
    }
    if (lane == 63) tmp[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += tmp[w];
    const int excl = before + v - sum;
#pragma unroll
    for (int j = 0; j < kPrefix / kThreads; ++j) {
      const int e = (kPrefix / kThreads) * t + j;
      if (e < G) pp[e + 1] = excl + c[j];
    }
    if (t == 0) pp[0] = 0;
    __syncthreads();  // pp complete; tmp free for the next problem
  }
}

// Largest e in [0, G) with pp[e] <= key, all 64 lanes searching at once
// (pp[0] = 0 <= key, and G <= kPrefix - 1 so every read stays inside the
// problem's prefix array).
__device__ __forceinline__ int find_expert(const int* pp, int G, int key, int lane) {
  int lo = 0;
  if (G > 64) {  // uniform: 64 segments of 16 experts, then one segment
    const int i = lane * 16;
    const uint64_t m = __builtin_amdgcn_ballot_w64(i < G && pp[i] <= key);
    lo = (63 - __builtin_clzll(m)) * 16;
    const int j = min(lo + lane, kPrefix - 1);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < 16 && j < G && pp[j] <= key);
    return uniform(lo + 63 - __builtin_clzll(m2));
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(lane < G && pp[lane] <= key);
  return uniform(63 - __builtin_clzll(m));
}

// A wave's position in its job sequence over one problem (all fields
// wave-uniform).
struct Cursor {
  int u;                 // unit of the problem (>= units: finished)
  int e, n0;             // expert and first weight row of the unit
  int c0, r1;            // the unit's token rows [c0, r1), at most 32
  int k;                 // current K slice (job) of kJobK elements
  uint32_t xq[2], xs[2]; // this lane's activation row offsets per token
                         // fragment (kOob: no row)
};

// Unit u of the problem (or the finished state past the last one).  Every
// field is stored once, on both paths, so the cursor stays in registers.
__device__ __forceinline__ void decode(ProblemRef P, const int* pp, int units, int u, int lane,
                                       Cursor& c) {
  int cu = units, e = 0, n0 = 0, c0 = 0, r1 = 0;
  if (u < units) {
    const int tiles = P.tiles;
    e = find_expert(pp, P.G, u / tiles, lane);
    const int p0 = uniform(pp[e]), ce = uniform(pp[e + 1]) - p0;
    if (ce > 0) {  // always, unless the offsets were inconsistent
      const int local = u - tiles * p0;
      const int t = min(max(local / ce, 0), tiles - 1), ch = local - t * ce;
      int64_t er0, er1;
      expert_rows(scalar_ptr(P.m_offsets), P.total_m, e, er0, er1);
      // rows stay inside the expert's clamped range whatever pp holds
      int64_t lo = er0 + 32 * (int64_t)ch;
      lo = lo < er0 ? er0 : (lo > er1 ? er1 : lo);
      cu = u;
      n0 = t * kRows;
      c0 = (int)lo;
      r1 = (int)(er1 < lo + 32 ? er1 : lo + 32);
    }
  }
  c.u = cu;
  c.e = e;
  c.n0 = n0;
  c.c0 = c0;
  c.r1 = r1;
  c.k = 0;
}

__device__ __forceinline__ void opaque(u32x4& v) { asm volatile("" : "+v"(v)); }

struct XFrags {
  u32x4 q[2][4];  // token fragments 0, 1: 64 nibble bytes each
  u32x2 s[2];     // their 8 scale bytes
};

// The units [first, first + stride, ...) of problem pi, through its own
// load/compute pipeline.  GATHER (the problem has a routing index): grouped
// row r reads activation row row_index[r] (an index outside [0, a_rows)
// reads as a zero row); otherwise grouped row r is activation row r.
template <bool GATHER>
__device__ __forceinline__ void run_problem(int pi, const int* pp, int units, int first,
                                            int stride, uint8_t* ring) {
  ProblemRef P = problem(pi);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int K = P.K;
  const uint32_t qrow = (uint32_t)(K / 2), srow = (uint32_t)(K / 16);
  const uint32_t wq_bytes = (uint32_t)P.N * qrow, ws_bytes = (uint32_t)P.N * srow;
  const uint32_t xq_bytes = (uint32_t)P.a_rows * qrow, xs_bytes = (uint32_t)P.a_rows * srow;
  const uint8_t* __restrict__ a_q = P.a_q;
  const uint8_t* __restrict__ a_s = P.a_s;
  const auto row_index = scalar_ptr(P.row_index);  // used with GATHER

  // Load offsets = a per-lane constant + a scalar per job.  Weight nibble
  // load k (16 B per lane) covers unit rows 4k .. 4k+3: lane L takes row
  // 4k + L/16 and physical 16-byte chunk L%16 of its 256-byte LDS row, which
  // holds logical chunk (L%16) ^ (row%16).  The scale load covers all 32 rows
  // (lane L: row L/2, half L%2).  Token fragment g holds chunk rows 16g+li.
  // Offsets stay in the range-checked vector operand, so weight rows past N
  // read as zero; token rows outside the unit's chunk get an out-of-range
  // offset (zero, and no memory traffic).
  uint32_t wq_lane[kNibLoads];
#pragma unroll
  for (int k = 0; k < kNibLoads; ++k) {
    const uint32_t row = 4u * k + (uint32_t)(lane >> 4);
    wq_lane[k] = row * qrow + (((uint32_t)(lane & 15) ^ (row & 15u)) << 4);
  }
  const uint32_t ws_lane = (uint32_t)(lane >> 1) * srow + (uint32_t)(lane & 1) * 16u;

  // Activation rows of the unit's chunk for this lane's two token fragments
  // (chunk rows 16g + li), as byte offsets of the row starts.  With a
  // routing index the chunk's 32 indices come through the scalar cache (so
  // their wait never drains the vector loads) and each lane picks its own.
  auto chunk_rows = [&](Cursor& c) {
    int src[2] = {c.c0 + li, c.c0 + 16 + li};
    if constexpr (GATHER) {
      const int base = uniform(c.c0);
      const int last = (int)P.total_m - 1;
      int v0 = 0, v1 = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i0 = row_index[min(base + j, last)], i1 = row_index[min(base + 16 + j, last)];
        v0 = li == j ? i0 : v0;
        v1 = li == j ? i1 : v1;
      }
      src[0] = v0;
      src[1] = v1;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bool ok = c.c0 + 16 * g + li < c.r1 && src[g] >= 0 && (int64_t)src[g] < P.a_rows;
      c.xq[g] = ok ? (uint32_t)src[g] * qrow : kOob;
      c.xs[g] = ok ? (uint32_t)src[g] * srow : kOob;
    }
  };

  auto advance = [&](Cursor& c) {
    if (c.u >= units) return;
    if (++c.k < P.nunits) return;
    decode(P, pp, units, c.u < units - stride ? c.u + stride : units, lane, c);
  };

  XFrags xs[kSlots];

  // The sources of the job at `c` (a finished wave reloads expert 0's first
  // slice as padding).
  struct JobSrc {
    const uint8_t* wq;
    const uint8_t* ws;
    uint32_t wq_job, ws_job;
  };
  auto job_src = [&](Cursor& c) {
    const bool live = c.u < units;
    if (live && c.k == 0) chunk_rows(c);  // uniform
    const int e = live ? c.e : 0;
    return JobSrc{P.b_q + (int64_t)e * P.N * qrow, P.b_s + (int64_t)e * P.N * srow,
                  live ? (uint32_t)c.n0 * qrow + (uint32_t)c.k * kRowNib : 0u,
                  live ? (uint32_t)c.n0 * srow + (uint32_t)c.k * kRowSc : 0u};
  };

  // Loads of the job at `c` into slot S: weights to LDS, activations to
  // registers, kLoadsPerJob memory instructions in two parts.  Part A (the
  // activations and the first kDmaA weight DMAs) goes out before the
  // previous job's products, part B (the other weight DMAs) after step
  // kStepB of them, so the wave does not stall on a burst of 28 loads
  // while the matrix core and the vector unit sit idle.
  auto issue_a = [&](Cursor& c, const JobSrc& js, auto sc) {
    constexpr int S = decltype(sc)::value;
    const bool live = c.u < units;
    const uint8_t* wq = js.wq;
    const uint32_t wq_job = js.wq_job;
    const uint32_t xq_job = (uint32_t)c.k * kRowNib + (uint32_t)lq * 64u;
    const uint32_t xs_job = (uint32_t)c.k * kRowSc + (uint32_t)lq * 8u;
    uint8_t* slot = ring + S * kSlotBytes;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // token rows outside the unit's chunk are not fetched at all
      const bool ok = live && c.xq[g] != kOob;
      const uint32_t qo = ok ? c.xq[g] + xq_job : kOob;
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[S].q[g][i] = ld16(a_q, xq_bytes, ok ? qo + 16u * i : kOob);
      xs[S].s[g] = ld8(a_s, xs_bytes, ok ? c.xs[g] + xs_job : kOob);
    }
#pragma unroll
    for (int k = 0; k < kDmaA; ++k) dma16(wq, wq_bytes, wq_job + wq_lane[k], slot + k * 1024);
  };
  auto issue_b = [&](const JobSrc& js, auto sc) {
    constexpr int S = decltype(sc)::value;
    uint8_t* slot = ring + S * kSlotBytes;
#pragma unroll
    for (int k = kDmaA; k < kNibLoads; ++k) dma16(js.wq, wq_bytes, js.wq_job + wq_lane[k], slot + k * 1024);
#pragma unroll
    for (int m = 0; m < kScLoads; ++m)
      dma16(js.ws, ws_bytes, js.ws_job + 32u * m * srow + ws_lane, slot + kSlotNib + m * 1024);
  };

  f32x4 acc[kFrags][2];
#pragma unroll
  for (int f = 0; f < kFrags; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[f][g] = f32x4{0, 0, 0, 0};

  // One job from slot S (its loads have landed), then the unit's epilogue
  // if this was its last slice.
  auto compute = [&](const Cursor& c, auto sc, auto&& part_b) {
    constexpr int S = decltype(sc)::value;
    const uint8_t* slot = ring + S * kSlotBytes;
    u32x4 w[kFrags][4];
    Scales sw[kFrags][2];
#pragma unroll
    for (int f = 0; f < kFrags; ++f) {
      const int row = 16 * f + li;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[f][i] = *reinterpret_cast<const u32x4*>(slot + row * kRowNib + (((4 * lq + i) ^ (row & 15)) << 4));
      const u32x2 s8 = *reinterpret_cast<const u32x2*>(slot + kSlotNib + row * kRowSc + lq * 8);
      sw[f][0] = to_scales(s8[0]);
      sw[f][1] = to_scales(s8[1]);
    }
    const Scales sx0[2] = {to_scales(xs[S].s[0][0]), to_scales(xs[S].s[0][1])};
    const int ntok = c.r1 - c.c0;
    // Step T (0..15) uses dword T of the lane's 64 bytes: block T/2, i.e.
    // scale pair word T/8, block (T/2) % 4 within it.  Software-pipelined:
    // the MFMAs of step T go out beside the dequantisation of step T+1, so
    // the matrix core and the vector unit overlap inside the one wave a
    // SIMD runs.
    auto run_steps = [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;  // token fragments (1 or 2)
      Scales sx1[2];
      if constexpr (NT == 2) {
        sx1[0] = to_scales(xs[S].s[1][0]);
        sx1[1] = to_scales(xs[S].s[1][1]);
      }
      auto dq = [&](auto tc, f16x8(&a)[kFrags], f16x8(&b)[2]) {
        constexpr int T = decltype(tc)::value, Q = T / 4, D = T % 4, H = T / 8, TT = T % 8;
        b[0] = dequant_step<TT>(xs[S].q[0][Q][D], sx0[H]);
        if constexpr (NT == 2) b[1] = dequant_step<TT>(xs[S].q[1][Q][D], sx1[H]);
#pragma unroll
        for (int f = 0; f < kFrags; ++f) a[f] = dequant_step<TT>(w[f][Q][D], sw[f][H]);
      };
      f16x8 a[kFrags], b[2];
      dq(std::integral_constant<int, 0>{}, a, b);
      static_for<16>([&](auto tc) {
        constexpr int T = decltype(tc)::value;
        f16x8 an[kFrags], bn[2];
        if constexpr (T + 1 < 16) dq(std::integral_constant<int, T + 1>{}, an, bn);
#pragma unroll
        for (int f = 0; f < kFrags; ++f) {
          acc[f][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[f], b[0], acc[f][0], 0, 0, 0);
          if constexpr (NT == 2)
            acc[f][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[f], b[1], acc[f][1], 0, 0, 0);
        }
        if constexpr (T + 1 < 16) {
#pragma unroll
          for (int f = 0; f < kFrags; ++f) a[f] = an[f];
          b[0] = bn[0];
          b[1] = bn[1];
        }
        if constexpr (T == kStepB) part_b();
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    if (ntok > 16) {  // wave-uniform
      // fresh copies of the shared operands, so the compiler cannot hoist
      // the two branches' common dequantisation above the branch (that
      // would keep all of it live at once)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int f = 0; f < kFrags; ++f) opaque(w[f][i]);
        opaque(xs[S].q[0][i]);
      }
      run_steps(std::integral_constant<int, 2>{});
    } else {
      run_steps(std::integral_constant<int, 1>{});
    }
    if (c.k == P.nunits - 1) {
      // acc[f][g] reg r: weight row n0 + 16f + 4*lq + r, token c0 + 16g + li
      const float alpha = scalar_ptr(P.a_g)[0] * scalar_ptr(P.b_g)[c.e];
      void* __restrict__ y = P.y;
      const int64_t ld_y = P.ld_y;
      const int y_dtype = P.y_dtype;
      if (P.y_bytes != 0 && c.n0 + kRows <= P.N) {  // uniform
        // the lane's four consecutive outputs of a token in one store;
        // tokens outside the chunk get an offset past the output (no write)
        const auto ry = rsrc(y, P.y_bytes);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int tok = 16 * g + li;
          const uint32_t row_off = (uint32_t)(c.c0 + tok) * (uint32_t)ld_y;
#pragma unroll
          for (int f = 0; f < kFrags; ++f) {
            const uint32_t el = row_off + (uint32_t)(c.n0 + 16 * f + 4 * lq);
            const f32x4 v = acc[f][g] * alpha;
            if (y_dtype == 0) {
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry,
                                                     tok < ntok ? el * 4u : kOob, 0, 0);
            } else {
              const u32x2 b = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2)),
                               __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2))};
              __builtin_amdgcn_raw_buffer_store_b64(b, ry, tok < ntok ? el * 2u : kOob, 0, 0);
            }
            acc[f][g] = f32x4{0, 0, 0, 0};
          }
        }
      } else {
#pragma unroll
        for (int f = 0; f < kFrags; ++f)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int tok = 16 * g + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int n = c.n0 + 16 * f + 4 * lq + r;
              if (tok < ntok && n < P.N)
                store_out(y, (int64_t)(c.c0 + tok) * ld_y + n, acc[f][g][r] * alpha, y_dtype);
            }
            acc[f][g] = f32x4{0, 0, 0, 0};
          }
      }
    }
  };

  Cursor lc, cc;
  decode(P, pp, units, first, lane, lc);
  if (lc.u >= units) return;  // nothing of this problem for the wave
  cc = lc;
  static_for<kSlots - 1>([&](auto sc) {
    const JobSrc js = job_src(lc);
    issue_a(lc, js, sc);
    issue_b(js, sc);
    advance(lc);
  });
  // jobs rotate through the slots; the loads of job j + kSlots - 1 go out
  // before job j waits for its own (the younger jobs may stay in flight)
  bool more = true;
  while (more) {
    static_for<kSlots>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      if (!more) return;
      constexpr int SN = (S + kSlots - 1) % kSlots;
      const JobSrc js = job_src(lc);
      issue_a(lc, js, std::integral_constant<int, SN>{});
      // every load before part A of the next job has landed
      wait_vmcnt<(kSlots - 2) * kLoadsPerJob + kLoadsA>();
      compute(cc, sc, [&] { issue_b(js, std::integral_constant<int, SN>{}); });
      advance(lc);
      advance(cc);
      more = cc.u < units;
    });
  }
  wait_vmcnt<0>();  // padding loads land before the next problem reuses the ring
}

// The waves of the grid walk the union of the problems' units with a fixed
// stride, problem by problem; each problem runs its own pipeline (drained
// between problems), so its operand descriptors stay in scalar registers.
// Waves are numbered XCD by XCD (workgroups go round-robin over the XCDs),
// so consecutive units -- the chunks of one weight tile -- run at the same
// time on one XCD and share its L2 for that tile.
__global__ __launch_bounds__(kThreads, kWaves / 4) void gemm_grouped_kernel(const Problems ps) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = uniform(threadIdx.x >> 6);
  int* const pref = reinterpret_cast<int*>(smem + kWaves * kWaveLds);
  build_prefixes(ps, pref, reinterpret_cast<int*>(smem));
  const int grid = gridDim.x, b = blockIdx.x;
  const int x = b % kXcds, i = b / kXcds;
  const int v = (x * (grid / kXcds) + min(x, grid % kXcds) + i) * kWaves + wave;
  const int stride = grid * kWaves;
  uint8_t* ring = smem + wave * kWaveLds;
  int base = 0;  // first global unit of problem pi
  for (int pi = 0; pi < ps.count; ++pi) {
    ProblemRef P = problem(pi);
    const int* pp = pref + pi * kPrefix;
    const int units = P.tiles * uniform(pp[P.G]);
    int first = (v - base) % stride;
    first += first < 0 ? stride : 0;
    if (P.row_index != nullptr)  // uniform
      run_problem<true>(pi, pp, units, first, stride, ring);
    else
      run_problem<false>(pi, pp, units, first, stride, ring);
    base += units;
  }
}

// Upper bound of a problem's units: each expert with tokens adds at most
// one partial chunk.
int64_t unit_bound(int64_t G, int64_t total_m, int64_t N) {
  const int64_t tiles = (N + kRows - 1) / kRows;
  return tiles * ((G < total_m ? G : total_m) + (total_m + 31) / 32);
}

}  // namespace

bool grouped_units_fit(int64_t G, int64_t total_m, int64_t N) {
  return unit_bound(G, total_m, N) < ((int64_t)1 << 29);
}

hipError_t launch_gemm_grouped_multi(int count, const GroupedProblem* probs, hipStream_t stream) {
  if (count < 1 || count > kMaxProblems) return hipErrorInvalidValue;
  static int num_cu = 0;  // compute units of the current device (one query per process)
  if (num_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    num_cu = n;
  }
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)gemm_grouped_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return attr;
  // Problems with more than kMaxGroups experts run as pieces of consecutive
  // experts (each piece reads only its own experts' rows); up to
  // kMaxProblems pieces go into one launch.
  Problems ps{};
  int64_t bound = 0;
  auto flush = [&]() -> hipError_t {
    if (ps.count == 0) return hipSuccess;
    int64_t grid = (bound + kWaves - 1) / kWaves;
    if (grid > num_cu) grid = num_cu;  // persistent: one workgroup per CU
    if (grid < 1) grid = 1;
    gemm_grouped_kernel<<<(unsigned)grid, kThreads, kLds, stream>>>(ps);
    ps = Problems{};
    bound = 0;
    return hipGetLastError();
  };
  for (int i = 0; i < count; ++i) {
    const GroupedProblem& g = probs[i];
    if (!grouped_units_fit(g.G, g.total_m, g.N)) return hipErrorInvalidValue;
    const int64_t tiles = (g.N + kRows - 1) / kRows;
    // whole 4-column groups of a row go out in one store when the rows are
    // aligned for it and the output's byte extent fits 32-bit offsets
    const int es = g.y_dtype == 0 ? 4 : 2;
    const int64_t extent = g.total_m > 0 ? ((g.total_m - 1) * g.ld_y + g.N) * es : 0;
    const bool aligned = (reinterpret_cast<uintptr_t>(g.y) % (4 * es)) == 0 && g.ld_y % 4 == 0;
    const uint32_t y_bytes = aligned && extent < (int64_t)0xFFFFFFF0 ? (uint32_t)extent : 0u;
    for (int64_t g0 = 0; g0 < g.G; g0 += kMaxGroups) {
      const int64_t ng = g.G - g0 < kMaxGroups ? g.G - g0 : kMaxGroups;
      if (ps.count == kMaxProblems) {
        const hipError_t err = flush();
        if (err != hipSuccess) return err;
      }
      ps.p[ps.count++] = Problem{
          g.m_offsets + g0, g.row_index, g.a.q, g.a.s, g.a.g,
          g.b.q + g0 * g.N * (g.K / 2), g.b.s + g0 * g.N * (g.K / 16), g.b.g + g0, g.y, g.ld_y,
          g.total_m, g.row_index != nullptr ? g.a_rows : g.total_m, (int)ng, (int)g.N, (int)g.K,
          (int)(g.K / kJobK), (int)tiles, g.y_dtype, y_bytes};
      bound += unit_bound(ng, g.total_m, g.N);
    }
  }
  return flush();
}

hipError_t launch_gemm_grouped(int32_t G, const int32_t* m_offsets, const int32_t* row_index,
                               int64_t total_m, int64_t a_rows, int64_t N, int64_t K,
                               PackedOperand a, PackedOperand b, void* y, int y_dtype,
                               int64_t ld_y, hipStream_t stream) {
  const GroupedProblem g{G, m_offsets, row_index, total_m, a_rows, N, K, a, b, y, y_dtype, ld_y};
  return launch_gemm_grouped_multi(1, &g, stream);
}

}  // namespace nvfp4
