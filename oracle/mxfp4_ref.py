"""Plain CPU oracle for the MXFP4 variant of the block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module; the HIP
library never calls it and shares nothing with it.  fp64 throughout, one
library matmul as the contraction.

Why it exists, and what fixes it
--------------------------------
The pages are about NVFP4; their only word on 4-bit density in general is
that FP4 packs twice the values of FP8 and four times those of FP16/BF16
(magik.net "The 3.7 PFLOPS Revelation", "Input Knowledge", item 2).  This
variant swaps NVFP4's 16-element E4M3 block scales for 32-element
power-of-two (E8M0) scales, the block shape gfx950's scaled FP4 matrix
instructions consume natively, to show the format's compute ceiling.  No
page defines it, so the readings below are the Open Compute Project
microscaling (MX) definition, restated; every function is pinned by
``tests/test_oracle_mxfp4.py`` against the mathematics of that definition
(bit fields, exact rational brute force), but its parity against the pages
is UNPINNED: they say nothing that could confirm or refute it.

M1  A block is 32 consecutive K-elements of a row; its scale byte is
    E8M0: value 2^(b - 127) for b = 0..254, NaN for b = 255.
M2  Elements are E2M1 nibbles exactly as in NVFP4 (codes 0..7 magnitudes
    {0, .5, 1, 1.5, 2, 3, 4, 6}, bit 3 the sign; element 2j of a row in the
    low nibble of byte j); scales a plain row-major [rows, K/32] array.
M3  Conversion of a block: E = floor(log2(amax_b)) - 2 (2 is the exponent
    of E2M1's largest value, 6 = 1.5 * 2^2), clamped to [-127, 127]; the
    scale byte is E + 127 and each element is the E2M1 rounding (nearest,
    ties to the even code, saturating at 6) of x / 2^E, which is exact.
M4  amax_b = 0 gives scale byte 0 and magnitude 0; a block holding a NaN
    or an infinity gives scale byte 255 and all nibbles 0.
M5  y[m, n] = sum_k A(m, k) B(n, k), A(m, k) = E2M1(nib) * 2^(b - 127):
    no per-tensor scale (the power-of-two scales carry the range).
"""
from __future__ import annotations

import numpy as np

from .nvfp4_ref import E2M1_TABLE, pack_nibbles, unpack_nibbles

MX_BLOCK = 32
E8M0_NAN = 255

# midpoints between consecutive E2M1 magnitudes (codes j and j+1)
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 byte -> fp64 2^(b - 127) (M1); NaN for 255."""
    b = np.asarray(codes, dtype=np.int64) & 0xFF
    return np.where(b == E8M0_NAN, np.nan, np.ldexp(1.0, b - 127))


def shared_exponent(amax) -> np.ndarray:
    """M3/M4: floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for 0.

    frexp writes amax = f * 2^e with f in [0.5, 1), so floor(log2 amax) is
    e - 1 exactly (no logarithm is evaluated).
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    E = np.where(amax > 0, e.astype(np.int64) - 1 - 2, -127)
    return np.clip(E, -127, 127)


def mxfp4_quantize_ref(x):
    """MXFP4 conversion of a 2-D array x [rows, K] (K % 32 == 0), M1-M4.

    Returns (q uint8 [rows, K/2], s uint8 [rows, K/32]).
    """
    x = np.asarray(x)
    assert x.ndim == 2 and x.shape[1] % MX_BLOCK == 0, x.shape
    xd = x.astype(np.float64)                       # exact for fp32 / bf16
    rows, cols = xd.shape
    nblk = cols // MX_BLOCK
    blocks = xd.reshape(rows, nblk, MX_BLOCK)
    finite = np.all(np.isfinite(blocks), axis=2)
    a = np.where(np.isfinite(blocks), np.abs(blocks), 0.0)
    amax = a.max(axis=2)
    E = shared_exponent(amax)                        # [rows, nblk]
    s = np.where(finite, E + 127, E8M0_NAN).astype(np.uint8)
    v = a / np.ldexp(1.0, E)[:, :, None]             # exact: power-of-two divisor
    code = np.zeros(v.shape, dtype=np.int64)         # nearest, ties to even code
    for j, t in enumerate(_E2M1_MID):
        code += ((v > t) | ((v == t) & (j % 2 == 1))).astype(np.int64)
    sign = np.signbit(blocks).astype(np.int64)
    nib = (sign << 3) | code
    nib = np.where(finite[:, :, None], nib, 0).astype(np.uint8).reshape(rows, cols)
    return pack_nibbles(nib), s


def mxfp4_dequantize_ref(q, s) -> np.ndarray:
    """Packed MXFP4 operand -> fp64 [rows, K] values (exact)."""
    nib = unpack_nibbles(q)
    return E2M1_TABLE[nib.astype(np.int64) & 15] * np.repeat(e8m0_decode(s), MX_BLOCK, axis=1)


def mxfp4_gemm_ref(a_q, a_s, b_q, b_s):
    """y[m, n] = sum_k A(m, k) * B(n, k) (M5), B stored [N, K].

    Returns (y, bound_base) in fp64, bound_base = sum_k |A(m, k) B(n, k)|,
    the quantity the tolerance is stated against (as for NVFP4).
    """
    xa = mxfp4_dequantize_ref(a_q, a_s)
    wb = mxfp4_dequantize_ref(b_q, b_s)
    return xa @ wb.T, np.abs(xa) @ np.abs(wb).T
