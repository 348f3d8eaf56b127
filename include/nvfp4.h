/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled GEMM library.
 *
 * Operation (kernelindex, "NVFP4 linear layer", description): y = x @ W^T,
 * where x [M, K] and W [N, K] are both FP4 (E2M1) values, each run of 16
 * consecutive K-elements of a row carrying one FP8 E4M3FN scale factor.
 * Layout (same page, workload line: in_features_half = K/2, sf_k = K/16,
 * sf_vec_size = 16; magik.net "The 3.7 PFLOPS Revelation", "Input Knowledge",
 * item 2: two FP4 values per byte, data K//2 wide, scales K//16 wide):
 *   q  uint8 [rows, K/2]   element 2j in the low nibble of byte j,
 *                          nibble = sign(bit 3) | E2M1 magnitude code (bits 0-2)
 *   s  uint8 [rows, K/16]  E4M3FN bit patterns, row-major, no swizzle
 *   g  fp32                per-tensor global scale; a row element decodes as
 *                          E2M1(nibble) * E4M3(s[row, k/16]) * g
 * Quantisation may run ahead of the GEMM and is timed apart from it
 * (leverageai "blackwell-nvfp4-gemm-optimization", "What is this?").
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers (HBM of the current HIP device),
 *     allocated and owned by the caller.  The library allocates, frees and
 *     synchronises nothing; it keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Results are valid once the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative status and touches no memory.  A
 *     failed kernel launch returns NVFP4_ERR_HIP.  No call aborts or throws.
 *   - Sizes of 0 are valid and enqueue nothing (NVFP4_OK).
 *   - Inputs must be finite and scale bytes must not be NaN (0x7F, 0xFF);
 *     this is documented, not checked (checking would cost a device pass).
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = -1, /* bad size, null pointer, bad stride / dtype  */
  NVFP4_ERR_UNSUPPORTED = -2, /* valid but unsupported (alignment, sizes)    */
  NVFP4_ERR_HIP = -3          /* a HIP runtime call or kernel launch failed */
} nvfp4_status;

typedef enum {
  NVFP4_F32 = 0,  /* IEEE binary32                                         */
  NVFP4_BF16 = 1  /* bfloat16, written round-to-nearest-even from the fp32
                     result; y_bf16 == RNE(y_f32) bit for bit              */
} nvfp4_dtype;

/* nvfp4_quantize flag: read *global_scale instead of computing it from the
 * data (static, ahead-of-time scale); the amax pass is skipped. */
#define NVFP4_GLOBAL_SCALE_GIVEN 1u

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_string(int status);

/* Library version as "major.minor.patch" (static string). */
const char* nvfp4_version(void);

/* Bytes of device workspace nvfp4_quantize needs for x of [rows, cols]
 * (partial maxima of the amax pass).  0 when rows*cols == 0. */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols);

/*
 * Quantise x [rows, cols] (row stride ld_x elements, dtype F32 or BF16) to
 * NVFP4: q [rows, cols/2], s [rows, cols/16] (both dense), *global_scale.
 *
 * Steps (exact reals, each stored quantity rounded once):
 *   g      = fl32(max|x| / 2688)                       (2688 = 448 * 6)
 *   s_b    = E4M3 nearest-even, saturating at 448, of max_{i in b}|x_i| / (6 g)
 *   code_i = E2M1 nearest-even, saturating at 6, of |x_i| / (E4M3(s_b) g)
 *   nibble = signbit(x_i) << 3 | code_i
 * A zero tensor gives g = 0, all scale bytes 0 and magnitude codes 0; a
 * block whose scale byte is 0 gets magnitude codes 0.  Output is unique:
 * the bytes equal the CPU definition exactly.
 *
 * Requirements: cols % 16 == 0; ld_x >= cols; x 16-byte aligned and
 * ld_x * sizeof(elem) % 16 == 0 (else NVFP4_ERR_UNSUPPORTED); q 8-byte
 * aligned.  workspace >= nvfp4_quantize_workspace_bytes(rows, cols) bytes,
 * 4-byte aligned (may be NULL when flags has NVFP4_GLOBAL_SCALE_GIVEN).
 * flags & NVFP4_GLOBAL_SCALE_GIVEN: *global_scale (device) is read, not
 * written; it must be finite and >= 0.
 */
int nvfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                   int64_t ld_x, uint8_t* q, uint8_t* s, float* global_scale,
                   unsigned flags, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * nvfp4_quantize for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as nvfp4_quantize, without the
 * workspace: the amax pass keeps its partial maxima (at most 4 KB) in a
 * device array of the library's own, one per GPU, held until the process
 * ends; the call allocates nothing.  Every call on one GPU shares that
 * array, so calls that overlap on a GPU (concurrent streams, other host
 * threads) race and must be ordered by the caller.  Shapes whose partial
 * maxima would not fit return NVFP4_ERR_UNSUPPORTED (none do: the amax
 * pass runs at most 1024 workgroups).  The first call on a device looks up
 * the array's address there (no allocation); a failure of that lookup
 * returns NVFP4_ERR_HIP.
 */
int nvfp4_quantize_noalloc(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, uint8_t* q, uint8_t* s, float* global_scale,
                           unsigned flags, void* stream);

/*
 * Dense NVFP4 GEMM (kernelindex, "NVFP4 linear layer"): for m < M, n < N
 *   y[m, n] = fl32(a_g * b_g) * sum_{k<K} A(m, k) * B(n, k)
 * with A(m, k) = E2M1(a_q nibble (m, k)) * E4M3(a_s[m, k/16]) and B the same
 * for b = W [N, K].  Products are formed exactly and accumulated in fp32;
 * |y - y_exact| <= 1e-5 * sum_k |x_k w_k| per element (plus one bf16 ulp for
 * BF16 output).  a_g and b_g are DEVICE pointers to one fp32 each, so a
 * quantise -> GEMM chain needs no host round-trip.
 *
 * a_q [M, K/2], a_s [M, K/16], b_q [N, K/2], b_s [N, K/16] are dense.
 * y [M, N] has row stride ld_y >= N elements of y_dtype.
 * Any M, N >= 0; K % 16 == 0.  Shapes are dispatched to a decode kernel
 * (M <= 128), an MFMA tile kernel, or a general kernel for unaligned K.
 */
int nvfp4_gemm(int64_t M, int64_t N, int64_t K,
               const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
               const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
               void* y, nvfp4_dtype y_dtype, int64_t ld_y, void* stream);

/*
 * Dense NVFP4 GEMM whose output is NVFP4 again: the next layer's input
 * quantisation done in this GEMM's epilogue with a static global scale fixed
 * ahead of time (leverageai "blackwell-nvfp4-gemm-optimization", "What is
 * this?": quantisation may happen before execution), so y never makes a
 * round trip through HBM in a wide type.
 *   y[m, n] = the fp32 value nvfp4_gemm stores with y_dtype NVFP4_F32
 *   (y_q, y_s) = the encoding of y by nvfp4_quantize's steps with g = *y_g
 *                (the bytes nvfp4_quantize with NVFP4_GLOBAL_SCALE_GIVEN
 *                would write from that fp32 y, exactly)
 * y_q [M, N/2] and y_s [M, N/16] are dense (row strides N/2 and N/16
 * bytes); y_q is 8-byte aligned.  y_g is a DEVICE fp32 scalar, read only;
 * it must be finite and >= 0 (0 gives scale bytes 0 and magnitude codes 0).
 * Values whose magnitude exceeds 2688 * g saturate (scale 448, code 6).
 * N % 16 == 0 (NVFP4_ERR_INVALID_ARG otherwise); the other requirements and
 * the kernel dispatch are those of nvfp4_gemm.
 */
int nvfp4_gemm_nvfp4_out(int64_t M, int64_t N, int64_t K,
                         const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                         const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                         uint8_t* y_q, uint8_t* y_s, const float* y_g, void* stream);

/*
 * Grouped (per-expert) NVFP4 GEMM for mixture-of-experts layers whose
 * experts each see a small, uneven number of tokens (magik.net "The Moment
 * of Synthesis", "The Reasoning Process": grouped GEMM is the lever for tiny
 * per-expert batches).  Rows of A are sorted by group: group e owns rows
 * [m_offsets[e], m_offsets[e+1]) and multiplies them by its own weight
 *   B_e = (b_q + e*N*K/2 [N, K/2], b_s + e*N*K/16 [N, K/16], b_g[e]).
 *   y[r, n] = fl32(*a_g * b_g[e]) * sum_k A(r, k) * B_e(n, k)
 * m_offsets: DEVICE int32 [G+1], non-decreasing, m_offsets[0] = 0,
 * m_offsets[G] = total_m (the host copy of the last entry).  Empty groups
 * are allowed.  b_g: DEVICE fp32 [G]; a_g: DEVICE fp32 scalar.
 * y [total_m, N] with row stride ld_y, rows in A's order.  K % 16 == 0.
 * Monotonicity of m_offsets is a documented precondition: rows outside
 * [0, total_m) are never read or written even if it is violated.
 */
int nvfp4_grouped_gemm(int32_t G, const int32_t* m_offsets, int64_t total_m,
                       int64_t N, int64_t K,
                       const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                       const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                       void* y, nvfp4_dtype y_dtype, int64_t ld_y, void* stream);

/*
 * The same grouped GEMM reading its activation rows through an index list
 * instead of a pre-gathered copy (the routing step of a mixture-of-experts
 * layer, "The Moment of Synthesis", "The Reasoning Process": tokens are sent
 * to their experts before the grouped GEMM).  Grouped row r (expert-sorted,
 * m_offsets as above) multiplies activation row row_index[r] of
 * a [a_rows, K/2] / [a_rows, K/16]; y [total_m, N] keeps the grouped order.
 * row_index: DEVICE int32 [total_m]; an index outside [0, a_rows) reads as a
 * row of zeros.  Indices may repeat (a token routed to several experts).
 * Otherwise as nvfp4_grouped_gemm (a_rows = total_m and row_index[r] = r give
 * the same result).  Errors: NVFP4_ERR_INVALID_ARG also for a_rows < 0 or a
 * null row_index with total_m > 0.
 */
int nvfp4_grouped_gemm_gather(int32_t G, const int32_t* m_offsets, const int32_t* row_index,
                              int64_t total_m, int64_t a_rows, int64_t N, int64_t K,
                              const uint8_t* a_q, const uint8_t* a_s, const float* a_g,
                              const uint8_t* b_q, const uint8_t* b_s, const float* b_g,
                              void* y, nvfp4_dtype y_dtype, int64_t ld_y, void* stream);

/*
 * Several independent grouped GEMMs in one launch.  A mixture-of-experts
 * layer runs its gate_up and down projections as grouped GEMMs over the
 * same routing ("The Moment of Synthesis", "The Reasoning Process":
 * grouping is the lever for tiny per-expert batches; "The Moment of
 * Recalibration", "The Broader Narrative Arc": persistent grouped kernels);
 * one persistent launch over the union of their (expert, weight tile) work
 * shares the launch ramp, the per-CU fill and the tail.  The projections
 * are independent here (each has its own activation; the operation between
 * them is outside this library).
 *
 * Each element of `problems` (a HOST array of `count` entries, 0 <= count
 * <= NVFP4_GROUPED_MAX_PROBLEMS) describes one call with exactly the
 * meaning of nvfp4_grouped_gemm (row_index == NULL) or
 * nvfp4_grouped_gemm_gather (row_index != NULL, a_rows = rows of a); with
 * row_index == NULL, a_rows must be 0 or total_m.  Results are those of
 * the separate calls, bit for bit.  Outputs of different problems must not
 * overlap.  Every problem is validated before anything is enqueued; any
 * error leaves all outputs untouched.  Problems the streaming kernel cannot
 * take (K % 512 != 0, unaligned rows, operands of 4 GiB or more) make the
 * call run each problem on its own.
 */
#define NVFP4_GROUPED_MAX_PROBLEMS 4

typedef struct {
  int32_t G;                  /* groups (experts)                                */
  const int32_t* m_offsets;   /* DEVICE int32 [G+1]                              */
  const int32_t* row_index;   /* DEVICE int32 [total_m], or NULL                 */
  int64_t total_m;            /* m_offsets[G]                                    */
  int64_t a_rows;             /* rows of a when row_index != NULL                */
  int64_t N, K;
  const uint8_t* a_q;         /* [a_rows, K/2]  (total_m rows without row_index) */
  const uint8_t* a_s;         /* [a_rows, K/16]                                  */
  const float* a_g;           /* DEVICE fp32 scalar                              */
  const uint8_t* b_q;         /* [G, N, K/2]                                     */
  const uint8_t* b_s;         /* [G, N, K/16]                                    */
  const float* b_g;           /* DEVICE fp32 [G]                                 */
  void* y;                    /* [total_m, N], row stride ld_y                   */
  nvfp4_dtype y_dtype;
  int64_t ld_y;
} nvfp4_grouped_problem;

int nvfp4_grouped_gemm_multi(int32_t count, const nvfp4_grouped_problem* problems,
                             void* stream);

/*
 * MXFP4 variant: 32-element blocks with power-of-two (E8M0) scales, the
 * block shape the gfx950 scaled FP4 matrix instruction consumes natively,
 * so the products need no dequantisation.  The pages define NVFP4 only
 * (FP4 packs twice the values of FP8 and four times those of FP16: magik.net
 * "The 3.7 PFLOPS Revelation", "Input Knowledge", item 2); this format
 * follows the microscaling definition and shows the 4-bit format's compute
 * ceiling on this hardware.
 *
 * nvfp4_mxfp4_quantize: x (fp32 | bf16) [rows, cols], row stride ld_x
 * elements -> q [rows, cols/2] (element 2j in the low nibble of byte j) and
 * s [rows, cols/32] E8M0 bytes (value 2^(b - 127); 255 is NaN), all DEVICE.
 * Per 32-element block: E = floor(log2(amax)) - 2 clamped to [-127, 127]
 * (-127 for a zero block), s = E + 127, each element the E2M1 rounding
 * (nearest, ties to the even code, saturating at 6, sign kept) of x / 2^E;
 * a block holding a NaN or an infinity gets s = 255 and zero nibbles.  One
 * pass, no workspace, deterministic.
 * Errors: NVFP4_ERR_INVALID_ARG for cols % 32 != 0, negative sizes, a bad
 * dtype, ld_x < cols or a null pointer with rows, cols > 0;
 * NVFP4_ERR_UNSUPPORTED for x or its rows not 16-byte aligned, q not
 * 16-byte aligned, or a dimension above 2^30.
 */
int nvfp4_mxfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                         int64_t ld_x, uint8_t* q, uint8_t* s, void* stream);

/*
 * y[m, n] = sum_k A(m, k) * B(n, k) with MXFP4 operands A = (a_q [M, K/2],
 * a_s [M, K/32]) and B = W = (b_q [N, K/2], b_s [N, K/32]), all DEVICE; no
 * per-tensor scale.  y [M, N] (fp32 or bf16, round to nearest even), row
 * stride ld_y.  fp32 accumulation; a NaN scale byte gives NaN outputs; terms
 * below fp32's subnormal range are lost.  K % 128 == 0 with 16-byte aligned
 * nibble rows and 4-byte aligned scale rows runs on the scaled FP4 matrix
 * instruction; other shapes run a general kernel.  K == 0 writes zeros.
 * Errors: NVFP4_ERR_INVALID_ARG for K % 32 != 0, negative sizes, a bad
 * y_dtype, ld_y < N or a null pointer; NVFP4_ERR_UNSUPPORTED for a
 * dimension above 2^30.
 */
int nvfp4_mxfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
                     const uint8_t* b_q, const uint8_t* b_s, void* y, nvfp4_dtype y_dtype,
                     int64_t ld_y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
