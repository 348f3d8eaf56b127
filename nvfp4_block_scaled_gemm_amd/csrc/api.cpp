// C ABI of the NVFP4 library (include/nvfp4.h): host-side argument checks and
// shape dispatch.  All checks run before anything is enqueued, so invalid
// calls return an error without touching the GPU.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include "nvfp4_dispatch.h"
#include "nvfp4_internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps 32-bit tile indexing safe

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Common checks of one packed operand [rows, K].
bool operand_ok(int64_t rows, int64_t K, const uint8_t* q, const uint8_t* s, const float* g) {
  if (rows == 0 || K == 0) return g != nullptr;
  return q != nullptr && s != nullptr && g != nullptr;
}

// Kernel eligibility for the tiled paths: 16-byte aligned nibble rows and
// 8-byte aligned scale rows.
bool tiled_ok(int64_t K, const uint8_t* q, const uint8_t* s, int64_t kmult) {
  return K % kmult == 0 && aligned(q, 16) && aligned(s, 8);
}

using nvfp4::offsets32_ok;

nvfp4::OperandAlign align_of(const uint8_t* q, const uint8_t* s) {
  return {aligned(q, 16), aligned(s, 8), aligned(s, 16)};
}

// Checks of one grouped problem (row_index == nullptr: rows of A are the
// grouped rows themselves, a_rows == total_m).  Returns NVFP4_OK, an error,
// or 1 for "valid, nothing to do".
int grouped_check(int32_t G, const int32_t* m_offsets, int64_t total_m, int64_t a_rows,
                  int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                  const uint8_t* b_q, const uint8_t* b_s, const float* b_g, const void* y,
                  nvfp4_dtype y_dtype, int64_t ld_y) {
  if (G < 0 || total_m < 0 || N < 0 || K < 0 || K % 16 != 0) return NVFP4_ERR_INVALID_ARG;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_ERR_INVALID_ARG;
  if (G == 0 && total_m != 0) return NVFP4_ERR_INVALID_ARG;
  if (total_m > kMaxDim || a_rows > kMaxDim || N > kMaxDim || K > kMaxDim)
    return NVFP4_ERR_UNSUPPORTED;
  if (total_m == 0 || N == 0) return 1;
  if (m_offsets == nullptr || y == nullptr || ld_y < N) return NVFP4_ERR_INVALID_ARG;
  if (!operand_ok(a_rows, K, a_q, a_s, a_g) || !operand_ok(N, K, b_q, b_s, b_g))
    return NVFP4_ERR_INVALID_ARG;
  return NVFP4_OK;
}

// The streaming grouped kernel takes K % 512 == 0, aligned rows, operands
// whose byte offsets fit 32 bits and unit counts that fit 32-bit ints;
// anything else runs the general kernel.
bool grouped_streams(const nvfp4::GroupedProblem& g) {
  return g.K > 0 && tiled_ok(g.K, g.a.q, g.a.s, 512) && tiled_ok(g.K, g.b.q, g.b.s, 512) &&
         offsets32_ok(g.total_m, g.K) && offsets32_ok(g.a_rows, g.K) && offsets32_ok(g.N, g.K) &&
         nvfp4::grouped_units_fit(g.G, g.total_m, g.N);
}

int grouped_run(const nvfp4::GroupedProblem& g, hipStream_t st) {
  if (grouped_streams(g)) return from_hip(nvfp4::launch_gemm_grouped_multi(1, &g, st));
  return from_hip(nvfp4::launch_gemm_grouped_generic(g.G, g.m_offsets, g.row_index, g.total_m,
                                                     g.a_rows, g.N, g.K, g.a, g.b, g.y, g.y_dtype,
                                                     g.ld_y, st));
}

// Shared body of the two grouped entry points.
int grouped_impl(int32_t G, const int32_t* m_offsets, const int32_t* row_index, int64_t total_m,
                 int64_t a_rows, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
                 const float* a_g, const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                 void* y, nvfp4_dtype y_dtype, int64_t ld_y, void* stream) {
  const int v = grouped_check(G, m_offsets, total_m, a_rows, N, K, a_q, a_s, a_g, b_q, b_s, b_g,
                              y, y_dtype, ld_y);
  if (v != NVFP4_OK) return v == 1 ? NVFP4_OK : v;
  const nvfp4::GroupedProblem g{G, m_offsets, row_index, total_m, a_rows, N, K,
                                nvfp4::PackedOperand{a_q, a_s, a_g},
                                nvfp4::PackedOperand{b_q, b_s, b_g}, y, (int)y_dtype, ld_y};
  return grouped_run(g, (hipStream_t)stream);
}

// Shape dispatch of the dense GEMM (both entry points, so an NVFP4 output
// sees exactly the fp32 values of the fp32 output).  dt 2: NVFP4 output qo.
int gemm_dispatch(int64_t M, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
                  const float* a_g, const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                  void* y, int dt, int64_t ld_y, nvfp4::QuantOut qo, hipStream_t st) {
  const nvfp4::PackedOperand a{a_q, a_s, a_g}, b{b_q, b_s, b_g};
  switch (nvfp4::gemm_path(M, N, K, align_of(a_q, a_s), align_of(b_q, b_s), dt == 2)) {
    case nvfp4::GemmPath::kDecodeRows:
      return from_hip(nvfp4::launch_gemm_decode_rows(M, N, K, a, b, y, dt, ld_y, st));
    case nvfp4::GemmPath::kDecodeLds:
      return from_hip(nvfp4::launch_gemm_decode_lds(M, N, K, a, b, y, dt, ld_y, st, qo));
    case nvfp4::GemmPath::kDecode:
      return from_hip(nvfp4::launch_gemm_decode(M, N, K, a, b, y, dt, ld_y, st, qo));
    case nvfp4::GemmPath::kMfma:
      return from_hip(nvfp4::launch_gemm_mfma(M, N, K, a, b, y, dt, ld_y, st, qo));
    default:
      return from_hip(nvfp4::launch_gemm_generic(M, N, K, a, b, y, dt, ld_y, st, qo));
  }
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_INVALID_ARG: return "NVFP4_ERR_INVALID_ARG";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP";
    default: return "NVFP4_UNKNOWN_STATUS";
  }
}

const char* nvfp4_version(void) { return "0.1.0"; }

size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return nvfp4::quantize_workspace_bytes(rows, cols);
}

int nvfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                   int64_t ld_x, uint8_t* q, uint8_t* s, float* global_scale, unsigned flags,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_INVALID_ARG;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_INVALID_ARG;
  if (flags & ~NVFP4_GLOBAL_SCALE_GIVEN) return NVFP4_ERR_INVALID_ARG;
  if (global_scale == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (rows > kMaxDim || cols > kMaxDim) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (ld_x < cols) return NVFP4_ERR_INVALID_ARG;
  const bool given = (flags & NVFP4_GLOBAL_SCALE_GIVEN) != 0;
  if (!given) {
    if (workspace == nullptr || !aligned(workspace, 4)) return NVFP4_ERR_INVALID_ARG;
    if (workspace_bytes < nvfp4::quantize_workspace_bytes(rows, cols))
      return NVFP4_ERR_INVALID_ARG;
  }
  const int64_t esz = x_dtype == NVFP4_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ld_x * esz) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(q, 8)) return NVFP4_ERR_UNSUPPORTED;
  return from_hip(nvfp4::launch_quantize(x, (int)x_dtype, rows, cols, ld_x, q, s, global_scale,
                                         given, workspace, (hipStream_t)stream));
}

int nvfp4_quantize_noalloc(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, uint8_t* q, uint8_t* s, float* global_scale,
                           unsigned flags, void* stream) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_INVALID_ARG;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_INVALID_ARG;
  if (flags & ~NVFP4_GLOBAL_SCALE_GIVEN) return NVFP4_ERR_INVALID_ARG;
  if (global_scale == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (rows > kMaxDim || cols > kMaxDim) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (ld_x < cols) return NVFP4_ERR_INVALID_ARG;
  const int64_t esz = x_dtype == NVFP4_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ld_x * esz) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(q, 8)) return NVFP4_ERR_UNSUPPORTED;
  const bool given = (flags & NVFP4_GLOBAL_SCALE_GIVEN) != 0;
  void* ws = nullptr;
  if (!given) {
    // the partial maxima must fit the library's array
    if (nvfp4::quantize_workspace_bytes(rows, cols) > nvfp4::quantize_scratch_bytes())
      return NVFP4_ERR_UNSUPPORTED;
    const int e = from_hip(nvfp4::quantize_scratch(&ws));
    if (e != NVFP4_OK) return e;
  }
  return from_hip(nvfp4::launch_quantize(x, (int)x_dtype, rows, cols, ld_x, q, s, global_scale,
                                         given, ws, (hipStream_t)stream));
}

int nvfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
               const float* a_g, const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
               void* y, nvfp4_dtype y_dtype, int64_t ld_y, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return NVFP4_ERR_INVALID_ARG;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return NVFP4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (y == nullptr || ld_y < N) return NVFP4_ERR_INVALID_ARG;
  if (!operand_ok(M, K, a_q, a_s, a_g) || !operand_ok(N, K, b_q, b_s, b_g))
    return NVFP4_ERR_INVALID_ARG;
  return gemm_dispatch(M, N, K, a_q, a_s, a_g, b_q, b_s, b_g, y, (int)y_dtype, ld_y,
                       nvfp4::QuantOut{}, (hipStream_t)stream);
}

int nvfp4_gemm_nvfp4_out(int64_t M, int64_t N, int64_t K, const uint8_t* a_q,
                         const uint8_t* a_s, const float* a_g, const uint8_t* b_q,
                         const uint8_t* b_s, const float* b_g, uint8_t* y_q, uint8_t* y_s,
                         const float* y_g, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || N % 16 != 0) return NVFP4_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return NVFP4_ERR_UNSUPPORTED;
  if (y_g == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (y_q == nullptr || y_s == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (!operand_ok(M, K, a_q, a_s, a_g) || !operand_ok(N, K, b_q, b_s, b_g))
    return NVFP4_ERR_INVALID_ARG;
  if (!aligned(y_q, 8)) return NVFP4_ERR_UNSUPPORTED;
  return gemm_dispatch(M, N, K, a_q, a_s, a_g, b_q, b_s, b_g, nullptr, 2, N,
                       nvfp4::QuantOut{y_q, y_s, y_g}, (hipStream_t)stream);
}

int nvfp4_grouped_gemm(int32_t G, const int32_t* m_offsets, int64_t total_m, int64_t N,
                       int64_t K, const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                       const uint8_t* b_q, const uint8_t* b_s, const float* b_g, void* y,
                       nvfp4_dtype y_dtype, int64_t ld_y, void* stream) {
  return grouped_impl(G, m_offsets, nullptr, total_m, total_m, N, K, a_q, a_s, a_g, b_q, b_s, b_g,
                      y, y_dtype, ld_y, stream);
}

int nvfp4_grouped_gemm_gather(int32_t G, const int32_t* m_offsets, const int32_t* row_index,
                              int64_t total_m, int64_t a_rows, int64_t N, int64_t K,
                              const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                              const uint8_t* b_q, const uint8_t* b_s, const float* b_g, void* y,
                              nvfp4_dtype y_dtype, int64_t ld_y, void* stream) {
  if (a_rows < 0) return NVFP4_ERR_INVALID_ARG;
  if (total_m > 0 && row_index == nullptr) return NVFP4_ERR_INVALID_ARG;
  return grouped_impl(G, m_offsets, row_index, total_m, a_rows, N, K, a_q, a_s, a_g, b_q, b_s, b_g,
                      y, y_dtype, ld_y, stream);
}

int nvfp4_grouped_gemm_multi(int32_t count, const nvfp4_grouped_problem* problems,
                             void* stream) {
  if (count < 0 || count > NVFP4_GROUPED_MAX_PROBLEMS) return NVFP4_ERR_INVALID_ARG;
  if (count == 0) return NVFP4_OK;
  if (problems == nullptr) return NVFP4_ERR_INVALID_ARG;
  nvfp4::GroupedProblem gs[NVFP4_GROUPED_MAX_PROBLEMS];
  int n = 0;
  bool all_stream = true;
  // every problem is checked before anything is enqueued
  for (int i = 0; i < count; ++i) {
    const nvfp4_grouped_problem& p = problems[i];
    const int64_t a_rows = p.row_index != nullptr ? p.a_rows : p.total_m;
    if (p.row_index != nullptr && p.a_rows < 0) return NVFP4_ERR_INVALID_ARG;
    if (p.row_index == nullptr && p.a_rows != 0 && p.a_rows != p.total_m)
      return NVFP4_ERR_INVALID_ARG;
    const int v = grouped_check(p.G, p.m_offsets, p.total_m, a_rows, p.N, p.K, p.a_q, p.a_s,
                                p.a_g, p.b_q, p.b_s, p.b_g, p.y, p.y_dtype, p.ld_y);
    if (v == 1) continue;  // valid, empty
    if (v != NVFP4_OK) return v;
    gs[n] = nvfp4::GroupedProblem{p.G, p.m_offsets, p.row_index, p.total_m, a_rows, p.N, p.K,
                                  nvfp4::PackedOperand{p.a_q, p.a_s, p.a_g},
                                  nvfp4::PackedOperand{p.b_q, p.b_s, p.b_g}, p.y,
                                  (int)p.y_dtype, p.ld_y};
    all_stream = all_stream && grouped_streams(gs[n]);
    ++n;
  }
  if (n == 0) return NVFP4_OK;
  const hipStream_t st = (hipStream_t)stream;
  if (all_stream) return from_hip(nvfp4::launch_gemm_grouped_multi(n, gs, st));
  for (int i = 0; i < n; ++i) {
    const int e = grouped_run(gs[i], st);
    if (e != NVFP4_OK) return e;
  }
  return NVFP4_OK;
}

int nvfp4_mxfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                         int64_t ld_x, uint8_t* q, uint8_t* s, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return NVFP4_ERR_INVALID_ARG;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_INVALID_ARG;
  if (rows > kMaxDim || cols > kMaxDim) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return NVFP4_ERR_INVALID_ARG;
  if (ld_x < cols) return NVFP4_ERR_INVALID_ARG;
  const int64_t esz = x_dtype == NVFP4_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ld_x * esz) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(q, 16)) return NVFP4_ERR_UNSUPPORTED;
  return from_hip(nvfp4::launch_mx_quantize(x, (int)x_dtype, rows, cols, ld_x, q, s,
                                            (hipStream_t)stream));
}

int nvfp4_mxfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
                     const uint8_t* b_q, const uint8_t* b_s, void* y, nvfp4_dtype y_dtype,
                     int64_t ld_y, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return NVFP4_ERR_INVALID_ARG;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return NVFP4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (y == nullptr || ld_y < N) return NVFP4_ERR_INVALID_ARG;
  if (K > 0 && (a_q == nullptr || a_s == nullptr || b_q == nullptr || b_s == nullptr))
    return NVFP4_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  // the matrix-core kernel: whole 128-element stages, 16-byte nibble rows,
  // 4-byte scale rows, operands (plus one tile of slack) under 4 GiB
  if (K > 0 && K % 128 == 0 && aligned(a_q, 16) && aligned(b_q, 16) && aligned(a_s, 4) &&
      aligned(b_s, 4) && offsets32_ok(M, K) && offsets32_ok(N, K))
    return from_hip(nvfp4::launch_gemm_mx_mfma(M, N, K, a_q, a_s, b_q, b_s, y, (int)y_dtype, ld_y,
                                               st));
  return from_hip(nvfp4::launch_mx_gemm_generic(M, N, K, a_q, a_s, b_q, b_s, y, (int)y_dtype,
                                                ld_y, st));
}

}  // extern "C"
