// Exact NVFP4 block encoder, shared by the quantiser and by the GEMM
// epilogues that write NVFP4 output (gfx950 only).
//
// Semantics (the pages leave them open; the reading taken is that every
// stored quantity is rounded once from its exact real value), for a block
// of 16 values with global scale g:
//   s_b    = nearest E4M3 (ties to even code, saturating at 448) to amax_b/(6g)
//   code_i = nearest E2M1 magnitude (ties to even, saturating at 6) to
//            |x_i| / (E4M3(s_b) * g); 0 when s_b == 0
//   nibble = signbit(x_i) << 3 | code_i
// Format: kernelindex "NVFP4 linear layer" (description: FP4 values with FP8
// E4M3FN scales per 16 elements); magik.net "The 3.7 PFLOPS Revelation",
// "Input Knowledge" item 2 (two values per byte).
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {
namespace enc {

// ---- loading one 16-element block as |x| bit patterns and sign bits -------

struct Block16 {
  float v[16];      // x_i as fp32 (exact for both input types), sign kept
};

__device__ __forceinline__ void load_block(const void* x, int dtype, int64_t elem_off,
                                           Block16& b) {
  if (dtype == 1) {  // bf16: two 16-byte loads
    const u32x4* p = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(x) + elem_off);
    u32x4 v0 = p[0], v1 = p[1];
    uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      b.v[2 * i] = __uint_as_float(w[i] << 16);
      b.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {  // fp32: four 16-byte loads
    const u32x4* p = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const float*>(x) + elem_off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = p[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) b.v[4 * j + i] = __uint_as_float(v[i]);
    }
  }
}

// The raw 32 (bf16) or 64 (fp32) bytes of one block, loaded ahead of use.
template <int DT>
struct RawBlock {
  u32x4 w[DT == 1 ? 2 : 4];
};

template <int DT>
__device__ __forceinline__ RawBlock<DT> load_raw(const void* x, int64_t elem_off) {
  RawBlock<DT> r;
  const u32x4* p = reinterpret_cast<const u32x4*>(
      reinterpret_cast<const uint8_t*>(x) + elem_off * (DT == 1 ? 2 : 4));
#pragma unroll
  for (int i = 0; i < (DT == 1 ? 2 : 4); ++i) r.w[i] = p[i];
  return r;
}

template <int DT>
__device__ __forceinline__ Block16 unpack(const RawBlock<DT>& r) {
  Block16 b;
  if constexpr (DT == 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = r.w[i >> 2][i & 3];
      b.v[2 * i] = __uint_as_float(w << 16);
      b.v[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) b.v[i] = __uint_as_float(r.w[i >> 2][i & 3]);
  }
  return b;
}

__device__ __forceinline__ uint32_t block_amax_bits(const Block16& b) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(b.v[i]) & 0x7FFFFFFFu);
  return m;  // non-negative floats order like their bit patterns
}

// Sign bits of the block moved to bit 3 of each nibble (elements 0-7 in
// `lo`, 8-15 in `hi`, element 2j in the low nibble of byte j).
__device__ __forceinline__ void sign_nibbles(const Block16& b, uint32_t& lo, uint32_t& hi) {
  lo = hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo |= (__float_as_uint(b.v[i]) >> 31) << (4 * i + 3);
    hi |= (__float_as_uint(b.v[8 + i]) >> 31) << (4 * i + 3);
  }
}

// Midpoint between E4M3 codes c and c+1 (c in 0..125) times 6, exactly:
// (E >= 1 ? 16 : 0) + 2m + 1 over 2^(11 - max(E,1)), E = c >> 3, m = c & 7.
__device__ __forceinline__ double e4m3_mid_times6(int c) {
  const int e = c >> 3, m = c & 7;
  const int mant = (e >= 1 ? 16 : 0) + 2 * m + 1;
  const int ex = (e >= 1 ? e : 1) - 11;
  return __builtin_ldexp((double)(6 * mant), ex);
}

// Exact value of E4M3 code c in 0..126.
__device__ __forceinline__ double e4m3_value(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? __builtin_ldexp((double)m, -9) : __builtin_ldexp((double)(8 + m), e - 10);
}

// Neighbours of a finite non-negative fp32 (bit pattern +-1; 0 steps up to
// the smallest subnormal).
__device__ __forceinline__ float next_up(float f) { return __uint_as_float(__float_as_uint(f) + 1u); }
__device__ __forceinline__ float next_down(float f) { return __uint_as_float(__float_as_uint(f) - 1u); }

// Largest fp32 <= t and smallest fp32 >= t, for finite non-negative t.
__device__ __forceinline__ float round_down_f32(double t) {
  float f = (float)t;
  if ((double)f > t) f = next_down(f);
  return f;
}
__device__ __forceinline__ float round_up_f32(double t) {
  float f = (float)t;
  if ((double)f < t) f = next_up(f);
  return f;
}

// A code within one step of the E4M3 code nearest to q >= 0 (q is the fp64
// product amax_b * (1 / 6g), whose relative error is far below the 1/16
// relative spacing of E4M3 midpoints).  Saturates at 0x7E.
__device__ __forceinline__ int e4m3_code_near(double q) {
  const int c_sub = (int)__builtin_rint(__builtin_fmin(q, 1.0) * 512.0);   // subnormals m * 2^-9
  int ex;
  const double fr = __builtin_frexp(q, &ex);                                // q = fr * 2^ex, fr in [0.5, 1)
  const int c_norm = ((ex + 6) << 3) + (int)__builtin_rint(fr * 16.0 - 8.0);
  const int c = q < 0x1p-6 ? c_sub : c_norm;
  return q < 448.0 ? (c < 126 ? c : 126) : 126;
}

// fp32 thresholds V_t (t = 0..6) with code = #{ t : |x| >= V_t } for a block
// of scale S (exact fp64 product E4M3 value * g):
//   odd t (a tie rounds up):   V_t = smallest fp32 >= mid_t * S
//   even t (a tie stays down): V_t = the fp32 just above the largest fp32 <= mid_t * S
__device__ __forceinline__ void thresholds_f64(double S, float (&V)[7]) {
  const double mid2[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
  for (int t = 0; t < 7; ++t) {
    const double u = mid2[t] * S;                     // exact
    V[t] = (t & 1) ? round_up_f32(u) : next_up(round_down_f32(u));
  }
}

// #{ t : a >= V_t } for non-decreasing V, by a three-level search.
__device__ __forceinline__ uint32_t e2m1_code(float a, const float (&V)[7]) {
  const bool h = a >= V[3];
  const bool h2 = a >= (h ? V[5] : V[1]);
  const float v3 = h ? (h2 ? V[6] : V[4]) : (h2 ? V[2] : V[0]);
  return (h ? 4u : 0u) + (h2 ? 2u : 0u) + (a >= v3 ? 1u : 0u);
}

// Per-tensor constants of the encode pass.
struct EncodeParams {
  float g;
  float inv6g_f;   // fl32(1 / (6g)), fast path only
  double gd, inv6g;
};

// The scale code is the number of E4M3 midpoints k (0..125) that
// amax_b / (6g) lies above, a tie counting only for odd k (so the result is
// even); the test compares with the exact fp64 product mid_k * 6 * g.
__device__ __forceinline__ bool above_mid(double amax_b, int k, double gd) {
  const double t = e4m3_mid_times6(k) * gd;
  return amax_b > t || (amax_b == t && (k & 1));
}

// Scale code of a block, g > 0: a candidate within one step of the answer
// (e4m3_code_near), then one exact test on each side.
__device__ __forceinline__ int scale_code(double amax_b, const EncodeParams& P) {
  const int c = e4m3_code_near(amax_b * P.inv6g);
  // above_mid is monotone in k, so at most one of the two corrections applies
  const bool down = c > 0 && !above_mid(amax_b, c > 0 ? c - 1 : 0, P.gd);
  const bool up = c < 126 && above_mid(amax_b, c, P.gd);
  return c - (down ? 1 : 0) + (up ? 1 : 0);
}

__device__ __forceinline__ float e4m3_value_f32(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf((float)(8 + m), e - 10);
}

// Nibbles of a block with scale code c > 0 by exact thresholds (fp64
// products; used when g is too small for the fp32 residual argument).
__device__ __forceinline__ void encode_exact(const Block16& b, int c, const EncodeParams& P,
                                             uint32_t& lo, uint32_t& hi) {
  float V[7];
  thresholds_f64((double)e4m3_value_f32(c) * P.gd, V);
  sign_nibbles(b, lo, hi);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo |= e2m1_code(__builtin_fabsf(b.v[i]), V) << (4 * i);
    hi |= e2m1_code(__builtin_fabsf(b.v[8 + i]), V) << (4 * i);
  }
}

// Encodes one block (16 values in b) to its 8 nibble bytes and scale byte.
//   kMode 0: g == 0 (every scale code 0, magnitudes 0)
//   kMode 1: 2^-88 <= g < 2^116 (fast path below)
//   kMode 2: any other g > 0 (exact thresholds through fp64 throughout)
template <int kMode>
__device__ __forceinline__ void encode_block(const Block16& b, const EncodeParams& P,
                                             uint8_t* __restrict__ qp, uint8_t* __restrict__ sp) {
  uint32_t lo_word, hi_word;
  int code_s = 0;
  if constexpr (kMode == 0) {
    sign_nibbles(b, lo_word, hi_word);
  } else {
    const float amax_f = __uint_as_float(block_amax_bits(b));
    if constexpr (kMode == 1) {
      // Scale code: the hardware E4M3 encoder (round to nearest, ties to
      // even; values above 464 would give NaN, hence the clamp to 448, which
      // the saturating rounding maps to anyway) on both ends of an interval
      // around amax_b / 6g, as for the elements below; the fp64 search
      // settles the rare block whose ends disagree.
      const float qv = amax_f * P.inv6g_f;
      const float qlo = __builtin_fminf(qv * (1.0f - 0x1p-20f), 448.0f);
      const float qhi = __builtin_fminf(qv * (1.0f + 0x1p-20f), 448.0f);
      const uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(qlo, qhi, 0, false);
      code_s = (int)(pk & 0xFF);
      if (code_s != (int)((pk >> 8) & 0xFF)) code_s = scale_code((double)amax_f, P);
    } else {
      code_s = scale_code((double)amax_f, P);
    }
    if constexpr (kMode == 1) {
      // Both ends of an interval around x_i / S go through the hardware E2M1
      // encoder (round to nearest, ties to the even code, saturating at 6,
      // sign kept).  The interval's half-width 2^-20 (relative) exceeds the
      // rounding error of the two products, so it contains the exact
      // quotient: when both ends encode alike, that code is the exact one;
      // otherwise a midpoint lies in the interval and the block takes the
      // exact threshold path.  A zero scale code gives magnitude 0.
      const float Sv = code_s != 0 ? e4m3_value_f32(code_s) : 1.0f;
      const float inv = __builtin_amdgcn_rcpf(Sv * P.g);
      const float mlo = inv * (1.0f - 0x1p-20f), mhi = inv * (1.0f + 0x1p-20f);
      uint32_t l0 = 0, l1 = 0, h0 = 0, h1 = 0;
      static_for<4>([&](auto pc) {
        constexpr int p = decltype(pc)::value;   // byte p <- elements 2p (low nibble), 2p + 1
        l0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l0, b.v[2 * p] * mlo, b.v[2 * p + 1] * mlo, 1.0f, p);
        h0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h0, b.v[2 * p] * mhi, b.v[2 * p + 1] * mhi, 1.0f, p);
        l1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l1, b.v[8 + 2 * p] * mlo, b.v[9 + 2 * p] * mlo, 1.0f, p);
        h1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h1, b.v[8 + 2 * p] * mhi, b.v[9 + 2 * p] * mhi, 1.0f, p);
        __builtin_amdgcn_sched_barrier(0);   // products just in time (fewer live registers)
      });
      const uint32_t sign_mask = 0x88888888u;
      lo_word = code_s != 0 ? l0 : (l0 & sign_mask);
      hi_word = code_s != 0 ? l1 : (l1 & sign_mask);
      // An element whose two ends disagree has exactly one E2M1 midpoint m
      // in its interval (midpoints lie >= 10 % apart), and its code is one of
      // the two ends'.  The quotient estimate rounded to two mantissa bits
      // is m; p = m * Sv is exact (<= 7 significant bits), and the sign of
      // r = fma(-p, g, |x|) = fl(|x| - p g) is that of the exact difference
      // (no underflow for g >= 2^-88), zero only on an exact tie, which goes
      // to the even code: the upper one for m in {0.75, 1.75, 3.5} (top
      // mantissa bit set), the lower one otherwise.  Only the element slots
      // in which some lane of the wave disagrees are visited.
      const uint32_t d0 = l0 ^ h0, d1 = l1 ^ h1;
      if (code_s != 0 && (d0 | d1) != 0) {
        static_for<16>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int sh = 4 * (i & 7);
          const uint32_t dw = i < 8 ? d0 : d1;
          if ((dw >> sh) & 0xFu) {
            const float a = __builtin_fabsf(b.v[i]);
            const float m = __uint_as_float((__float_as_uint(a * inv) + 0x00100000u) & 0xFFE00000u);
            const float r = __builtin_fmaf(-(m * Sv), P.g, a);
            const bool up = r > 0.0f || (r == 0.0f && ((__float_as_uint(m) >> 22) & 1u));
            if (up) {
              if (i < 8) lo_word = (lo_word & ~(0xFu << sh)) | (h0 & (0xFu << sh));
              else hi_word = (hi_word & ~(0xFu << sh)) | (h1 & (0xFu << sh));
            }
          }
        });
      }
    } else {
      if (code_s != 0) encode_exact(b, code_s, P, lo_word, hi_word);
      else sign_nibbles(b, lo_word, hi_word);
    }
  }
  u32x2 packed = {lo_word, hi_word};
  *reinterpret_cast<u32x2*>(qp) = packed;
  *sp = (uint8_t)code_s;
}

// Encode constants of a tensor with global scale g.
__device__ __forceinline__ EncodeParams make_params(float g) {
  EncodeParams P;
  P.g = g;
  P.gd = (double)g;
  P.inv6g = P.gd > 0.0 ? 1.0 / (6.0 * P.gd) : 0.0;
  P.inv6g_f = (float)P.inv6g;
  return P;
}

// encode_block's mode for global scale g: 0 for g == 0; 1 for
// 2^-88 <= g < 2^116; 2 (exact fp64 thresholds) for the scales outside.
// The fast mode needs fl32(1 / 6g) and fl32(1 / (E4M3(s) g)) to be normal
// fp32 numbers, so that their relative error stays far inside the 2^-20
// half-width of its intervals: E4M3(s) <= 448 < 2^9, so g < 2^116 keeps
// E4M3(s) g below 2^125 and 6g below 2^119; below 2^-88 the residual
// products underflow instead.
__device__ __forceinline__ int encode_mode(float g) {
  return !(g > 0.0f) ? 0 : ((g >= 0x1p-88f && g < 0x1p116f) ? 1 : 2);
}

}  // namespace enc
}  // namespace nvfp4
