"""Plain CPU oracle for the NVFP4 block-scaled GEMM  y = x . W^T.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP
library never calls it, and it shares no code, tables or helpers with the
HIP library (``nvfp4_block_scaled_gemm_amd``).  It is deliberately slow and
written to be checked by eye: fp64 everywhere, one library matmul as the
contraction, no blocking, fusion or reordering.

What the pages fix
------------------
* kernelindex, "NVFP4 linear layer" (description): y = x @ W^T, both x and W
  quantised to FP4, with FP8 E4M3FN scale factors, one per 16 elements.
* same page, "Current records", workload line: in_features = 8192,
  in_features_half = 4096, sf_k = 512, sf_vec_size = 16; i.e. packed data
  rows are K/2 bytes and scale rows K/16 bytes.
* magik.net "The 3.7 PFLOPS Revelation", section "Input Knowledge", item 2:
  FP4 values are packed two per byte, data tensors are K//2 wide and scale
  tensors K//16 wide.
* leverageai "blackwell-nvfp4-gemm-optimization", "What is this?":
  quantisation may happen ahead of execution and is timed apart from the GEMM.

Readings where the pages are silent (each is listed in the design doc)
----------------------------------------------------------------
R1  E2M1 magnitudes are {0, .5, 1, 1.5, 2, 3, 4, 6} for codes 0..7 (bits 0-2
    of a nibble), bit 3 is the sign.
R2  E4M3FN: sign bit 7, exponent bits 6-3 (bias 7), mantissa bits 2-0;
    exponent 0 is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; max 448.
R3  Global scale g = fl32(amax(|x|) / (448 * 6)), an fp32 decode multiplier:
    value ~= E2M1 * E4M3 * g.
R4  Block scale byte = E4M3 rounding of the exact quotient amax_b / (6 g),
    nearest value, ties to the even code, saturating at 448, never NaN.
R5  Element code = E2M1 rounding of the exact quotient |x| / (E4M3(s) * g),
    nearest magnitude, ties to the even code, saturating at 6.
R6  Every stored quantity is rounded once, from the exact real value.
R7  The sign nibble bit is the IEEE sign bit of x (so -0.0 gives 0x8).
R8  A zero tensor gives g = 0, scale bytes 0 and magnitude 0; a block whose
    scale byte is 0 has all magnitudes 0.
R9  Element 2j of a row is the low nibble of byte j; scales are a plain
    row-major [rows, K/16] array (no swizzle).
R10 W is stored [N, K] (out_features x in_features), y = x @ W^T.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against facts that do not come from this file
(bit-field derivations, torch's float8_e4m3fn decoder, exact rational brute
force with ``fractions.Fraction``, closed-form GEMM results, and the page's
workload parameters stored under ``tests/golden/``).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# decoders (R1, R2)
# ---------------------------------------------------------------------------

#: magnitude of an E2M1 code c = nibble & 7  (R1)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

#: 16-entry nibble -> value table: codes 0..7 positive, 8..15 negative
E2M1_TABLE = np.concatenate([E2M1_MAGNITUDES, -E2M1_MAGNITUDES])

E4M3_MAX = 448.0
GLOBAL_DIVISOR = 448.0 * 6.0   # 2688 (R3)


def e2m1_decode(nibbles) -> np.ndarray:
    """Nibble values 0..15 -> fp64 through the 16-entry table (R1)."""
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.int64) & 15]


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN byte -> fp64 from its bit fields (R2); NaN for 0x7F/0xFF."""
    b = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64) / 8.0, -6),
                   np.ldexp(1.0 + m.astype(np.float64) / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# finite non-negative E4M3 values, codes 0..126 (0x7E = 448)
_E4M3_POS = e4m3_decode(np.arange(127))
# midpoints between consecutive codes c and c+1, c = 0..125 (exact in fp64)
_E4M3_MID = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2.0
# midpoints between consecutive E2M1 magnitudes, j = 0..6
_E2M1_MID = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0


# ---------------------------------------------------------------------------
# packing (R9)
# ---------------------------------------------------------------------------

def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[rows, K] nibbles -> [rows, K/2] bytes, element 2j in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] nibbles (inverse of pack_nibbles)."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = q & 0x0F
    out[:, 1::2] = q >> 4
    return out


# ---------------------------------------------------------------------------
# quantiser (R3..R8), an encoding, so written step by step
# ---------------------------------------------------------------------------

def global_scale_ref(x) -> np.float32:
    """Step 2 (R3): g = fl32(amax_t / 2688) with IEEE fp32 division."""
    x = np.asarray(x)
    amax_t = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    return np.float32(amax_t / np.float32(GLOBAL_DIVISOR))


def _round_to_grid(value_vs: np.ndarray, thresholds_fn, n_mid: int) -> np.ndarray:
    """Round to nearest, ties to even code, by counting midpoints below.

    ``thresholds_fn(j)`` gives, for every element, the (exact) real midpoint
    between code j and code j+1 on the element's own scale.  The result code
    is the number of midpoints the value lies above; a value exactly on the
    midpoint between codes j and j+1 moves up only when j is odd (so the
    chosen code, j+1, is even).
    """
    code = np.zeros(value_vs.shape, dtype=np.int64)
    for j in range(n_mid):
        t = thresholds_fn(j)
        up = (value_vs > t) | ((value_vs == t) & (j % 2 == 1))
        code += up.astype(np.int64)
    return code


def quantize_ref(x, global_scale=None):
    """NVFP4 quantisation of a 2-D array x [rows, K] (K % 16 == 0).

    Returns (q uint8 [rows, K/2], s uint8 [rows, K/16], g np.float32).
    ``global_scale`` given: use it instead of step 2 (ahead-of-time scale).
    """
    x = np.asarray(x)
    assert x.ndim == 2 and x.shape[1] % 16 == 0, x.shape
    xd = x.astype(np.float64)                      # step 1: exact for fp32/bf16
    assert np.all(np.isfinite(xd)), "inputs must be finite"
    rows, cols = xd.shape
    nblk = cols // 16

    g = global_scale_ref(x) if global_scale is None else np.float32(global_scale)
    gd = float(g)
    blocks = xd.reshape(rows, nblk, 16)
    a = np.abs(blocks)
    sign = np.signbit(blocks).astype(np.uint8)     # R7

    if gd == 0.0:                                  # step 3 / R8
        s = np.zeros((rows, nblk), dtype=np.uint8)
        nib = (sign << 3).reshape(rows, cols)
        return pack_nibbles(nib), s, g

    # step 4 (R4): scale code from the exact quotient amax_b / (6 g); compare
    # amax_b with midpoint * 6 * g, a product of at most 31 significant bits,
    # so exact in fp64.
    amax_b = a.max(axis=2)
    s_code = _round_to_grid(amax_b, lambda c: _E4M3_MID[c] * 6.0 * gd, len(_E4M3_MID))
    s = s_code.astype(np.uint8)                    # 0..126, never NaN

    # step 5: block decode scale S_b = E4M3(s_b) * g (exact in fp64)
    S = _E4M3_POS[s_code] * gd                     # [rows, nblk]

    # step 6 (R5): element code from |x| / S_b; compare |x| with mid * S_b
    Sb = S[:, :, None]
    mag = _round_to_grid(a, lambda j: _E2M1_MID[j] * Sb, len(_E2M1_MID))
    mag = np.where(Sb == 0.0, 0, mag)              # R8: zero scale -> zero
    nib = ((sign << 3) | mag.astype(np.uint8)).reshape(rows, cols)
    return pack_nibbles(nib), s, g                 # step 7 (R9)


# ---------------------------------------------------------------------------
# GEMM (plain definition)
# ---------------------------------------------------------------------------

def dequantize_ref(q, s) -> np.ndarray:
    """Packed operand -> fp64 [rows, K] values E2M1(nib) * E4M3(scale).

    The per-tensor global scale is left out; every value is exact in fp64.
    """
    nib = unpack_nibbles(q)
    scale = np.repeat(e4m3_decode(s), 16, axis=1)
    return e2m1_decode(nib) * scale


def gemm_ref(a_q, a_s, a_g, b_q, b_s, b_g):
    """y[m, n] = ga * gb * sum_k A(m, k) * B(n, k)  (R10: B is W, [N, K]).

    Returns (y, bound_base) in fp64, where
    bound_base[m, n] = |ga * gb| * sum_k |A(m, k) * B(n, k)|, the per-element
    quantity the tolerance is stated against.
    """
    xa = dequantize_ref(a_q, a_s)
    wb = dequantize_ref(b_q, b_s)
    alpha = float(np.float64(a_g) * np.float64(b_g))
    y = (xa @ wb.T) * alpha
    bound = (np.abs(xa) @ np.abs(wb).T) * abs(alpha)
    return y, bound


def grouped_gemm_ref(m_offsets, a_q, a_s, a_g, b_q, b_s, b_g):
    """Per-group GEMMs over expert-sorted rows.

    Group e owns rows [m_offsets[e], m_offsets[e+1]) of A and uses weight
    b_q[e], b_s[e], b_g[e]; output rows keep A's row order.  Empty groups
    produce no rows.
    """
    off = np.asarray(m_offsets, dtype=np.int64)
    G = len(off) - 1
    N = b_q.shape[1]
    total = int(off[-1])
    y = np.zeros((total, N), dtype=np.float64)
    bound = np.zeros((total, N), dtype=np.float64)
    for e in range(G):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        y[r0:r1], bound[r0:r1] = gemm_ref(a_q[r0:r1], a_s[r0:r1], a_g,
                                          b_q[e], b_s[e], b_g[e])
    return y, bound


# ---------------------------------------------------------------------------
# tolerance
# ---------------------------------------------------------------------------

REL_TOL = 1e-5


def ulp_bf16(v) -> np.ndarray:
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7); 0 at v = 0."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    out = np.zeros_like(v)
    nz = v > 0
    out[nz] = np.ldexp(1.0, np.floor(np.log2(v[nz])).astype(np.int64) - 7)
    return out


def tolerance(y_ref, bound_base, out_dtype: str) -> np.ndarray:
    """Allowed |y - y_ref| per element: 1e-5 * sum|x w|, plus one bf16 ulp of
    y_ref when the output is bf16."""
    tol = REL_TOL * np.asarray(bound_base, dtype=np.float64)
    if out_dtype == "bf16":
        tol = tol + ulp_bf16(y_ref)
    return tol


def check_gemm(y, y_ref, bound_base, out_dtype: str):
    """Returns (ok, worst normalised error) for a GEMM result."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    tol = tolerance(y_ref, bound_base, out_dtype)
    ok = bool(np.all(err <= tol))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    return ok, float(ratio.max()) if ratio.size else 0.0
