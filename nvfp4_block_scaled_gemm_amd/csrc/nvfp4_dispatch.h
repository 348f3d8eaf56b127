// Shape -> kernel choice of the dense NVFP4 GEMM.  Host-only and free of HIP
// so that the predicate compiles (and is tested) with a plain C++ compiler.
//
// Every kernel addresses its operands through 32-bit buffer offsets, so each
// path also checks that the rows it reads in one launch stay below 4 GiB.
#pragma once

#include <stdint.h>

namespace nvfp4 {

enum class GemmPath : int {
  kDecodeLds = 0,  // up to 32 tokens, K % 1024 == 0: LDS-ring weight stream
  kDecodeRows = 4, // up to 4 tokens, K = 8192: whole-row weight stream
  kDecode = 1,     // up to 128 rows in 64-row passes, K % 256 == 0
  kMfma = 2,       // MFMA tiles, K % 128 == 0
  kGeneric = 3,    // any shape (one thread per output)
};

// Alignment facts of one packed operand: nibble rows start 16-byte aligned
// (q base), scale base 8- and 16-byte aligned.
struct OperandAlign {
  bool q16, s8, s16;
};

// Rows [0, rows) of a packed operand, plus up to 32 rows of slack that the
// tile kernels may address past the end, fit 32-bit byte offsets.
inline bool offsets32_ok(int64_t rows, int64_t K) {
  return (rows + 32) * (K / 2) < ((int64_t)1 << 32) - 16;
}

// Exactly rows x K/2 bytes (no slack) fit a 32-bit buffer range that still
// leaves room for the out-of-range offset the kernels use for "no row".
inline bool bytes32_ok(int64_t rows, int64_t K) {
  return rows * (K / 2) < ((int64_t)1 << 32) - 16;
}

// Token counts and K the whole-row decode kernel is built for (its
// activation operand lives in registers, unrolled over K).
inline bool decode_rows_shape(int64_t M, int64_t K) { return M >= 1 && M <= 4 && K == 8192; }

// nvfp4_out: the output is written as NVFP4 (encoded 16 columns at a time).
inline GemmPath gemm_path(int64_t M, int64_t N, int64_t K, OperandAlign a, OperandAlign b,
                          bool nvfp4_out = false) {
  if (K <= 0) return GemmPath::kGeneric;  // empty sum: the general kernel writes zeros
  const bool q_ok = a.q16 && b.q16;
  if (!nvfp4_out && decode_rows_shape(M, K) && q_ok && a.s16 && b.s16 && bytes32_ok(N, K) &&
      bytes32_ok(M, K))
    return GemmPath::kDecodeRows;
  // 16-byte scale loads at 64-byte row strides (K % 1024 == 0).
  if (M <= 32 && K % 1024 == 0 && q_ok && a.s16 && b.s16 && bytes32_ok(N, K) &&
      bytes32_ok(M, K))
    return GemmPath::kDecodeLds;
  // 97-128 rows go to the MFMA kernel's 64 x 64 tiles when those fill the
  // chip (one pass over W, ~38 us at N = K = 8192 whatever M), else to the
  // decode kernel's two 64-row passes, whose second pass costs less the
  // fewer rows it has.  Each decode pass reads at most 64 activation rows.
  const bool mid_mfma = M > 96 && ((M + 63) / 64) * ((N + 63) / 64) >= 256;
  const int64_t pass_rows = M < 64 ? M : 64;
  if (M <= 128 && !mid_mfma && K % 256 == 0 && q_ok && a.s8 && b.s8 && offsets32_ok(N, K) &&
      offsets32_ok(pass_rows, K))
    return GemmPath::kDecode;
  if (K % 128 == 0 && q_ok && a.s8 && b.s8 && offsets32_ok(M, K) && offsets32_ok(N, K))
    return GemmPath::kMfma;
  return GemmPath::kGeneric;
}

}  // namespace nvfp4
