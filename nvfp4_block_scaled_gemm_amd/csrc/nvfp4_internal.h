// Host-side launchers shared between the C ABI (api.cpp) and the kernel files.
// Every launcher assumes its arguments were validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace nvfp4 {

// quantize.hip
size_t quantize_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* q, uint8_t* s, float* gscale, bool scale_given,
                           void* workspace, hipStream_t stream);
// The library's own quantise workspace (a device array, one per GPU): its
// size in bytes, and its address on the current device (found once per
// device with hipGetSymbolAddress).
size_t quantize_scratch_bytes();
hipError_t quantize_scratch(void** ptr);

// Operand description of one packed NVFP4 matrix [rows, K].
struct PackedOperand {
  const uint8_t* q;  // [rows, K/2]
  const uint8_t* s;  // [rows, K/16]
  const float* g;    // device scalar (or [G] for grouped weights)
};

// NVFP4 output of a dense GEMM (y_dtype 2): y quantised with the given
// global scale *g (device fp32) into q [M, N/2] and s [M, N/16] (row-major,
// contiguous, N % 16 == 0, q 8-byte aligned), from the same fp32 values
// y_dtype 0 would store.
struct QuantOut {
  uint8_t* q;
  uint8_t* s;
  const float* g;
};

// gemm_generic.hip: any M, N, K % 16 == 0.
hipError_t launch_gemm_generic(int64_t M, int64_t N, int64_t K, PackedOperand a,
                               PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                               hipStream_t stream, QuantOut qo = {});

// row_index (nullptr: none): grouped row r reads activation row row_index[r]
// of the a_rows rows of `a`; an index outside [0, a_rows) reads as zeros.
hipError_t launch_gemm_grouped_generic(int32_t G, const int32_t* m_offsets,
                                       const int32_t* row_index, int64_t total_m, int64_t a_rows,
                                       int64_t N, int64_t K, PackedOperand a, PackedOperand b,
                                       void* y, int y_dtype, int64_t ld_y, hipStream_t stream);

// mxfp4.hip: MXFP4 conversion (cols % 32 == 0, 16-byte aligned x rows and
// q) and the general MXFP4 GEMM (any M, N, K % 32 == 0).
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t* q, uint8_t* s, hipStream_t stream);
hipError_t launch_mx_gemm_generic(int64_t M, int64_t N, int64_t K, const uint8_t* a_q,
                                  const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                                  void* y, int y_dtype, int64_t ld_y, hipStream_t stream);
// gemm_mfma.hip: MXFP4 on the scaled FP4 matrix instruction; K % 128 == 0,
// 16-byte aligned nibble rows, 4-byte aligned scale rows.
hipError_t launch_gemm_mx_mfma(int64_t M, int64_t N, int64_t K, const uint8_t* a_q,
                               const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                               void* y, int y_dtype, int64_t ld_y, hipStream_t stream);

// gemm_mfma.hip: K % 128 == 0, 16-byte aligned operand rows.
hipError_t launch_gemm_mfma(int64_t M, int64_t N, int64_t K, PackedOperand a,
                            PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                            hipStream_t stream, QuantOut qo = {});

// gemm_decode_lds.hip: M <= 32, K % 1024 == 0, 16-byte aligned nibble and
// scale bases, both operands' bytes < 4 GiB.
hipError_t launch_gemm_decode_lds(int64_t M, int64_t N, int64_t K, PackedOperand a,
                                  PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                                  hipStream_t stream, QuantOut qo = {});

// gemm_decode_rows.hip: whole-row weight stream for the shapes
// decode_rows_shape (nvfp4_dispatch.h) accepts, fp32 / bf16 output only;
// 16-byte aligned nibble and scale bases, both operands' bytes < 4 GiB.
hipError_t launch_gemm_decode_rows(int64_t M, int64_t N, int64_t K, PackedOperand a,
                                   PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                                   hipStream_t stream);

// gemm_skinny.hip: M <= 128 (decode; 64-row passes), K % 256 == 0, N * K / 2 < 4 GiB.
hipError_t launch_gemm_decode(int64_t M, int64_t N, int64_t K, PackedOperand a,
                              PackedOperand b, void* y, int y_dtype, int64_t ld_y,
                              hipStream_t stream, QuantOut qo = {});

// One grouped GEMM of a launch (row_index as above; a_rows is used only with
// a row_index).
struct GroupedProblem {
  int32_t G;
  const int32_t* m_offsets;
  const int32_t* row_index;
  int64_t total_m, a_rows, N, K;
  PackedOperand a, b;
  void* y;
  int y_dtype;
  int64_t ld_y;
};
constexpr int kGroupedMaxProblems = 4;  // = NVFP4_GROUPED_MAX_PROBLEMS

// gemm_grouped.hip: 1..kGroupedMaxProblems problems in one persistent launch,
// each with K % 512 == 0 and operands < 4 GiB.
hipError_t launch_gemm_grouped_multi(int count, const GroupedProblem* probs, hipStream_t stream);
// The streaming grouped kernel numbers its work units with 32-bit ints:
// true when a problem of this size fits.
bool grouped_units_fit(int64_t G, int64_t total_m, int64_t N);

// gemm_grouped.hip: K % 512 == 0, operands < 4 GiB; row_index as above.
hipError_t launch_gemm_grouped(int32_t G, const int32_t* m_offsets, const int32_t* row_index,
                               int64_t total_m, int64_t a_rows, int64_t N, int64_t K,
                               PackedOperand a, PackedOperand b, void* y, int y_dtype,
                               int64_t ld_y, hipStream_t stream);

}  // namespace nvfp4
