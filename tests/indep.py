"""Independent reference pieces for pinning the oracle (CPU only).

Nothing here imports the oracle.  E4M3 values come from torch's
``float8_e4m3fn`` decoder, E2M1 values from the bit-field formula (exponent
bias 1), and rounding from exact ``fractions.Fraction`` distance comparisons,
so a mistake in the oracle's table, midpoint counting or packing shows up as
a disagreement.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def e4m3_fraction(code: int) -> Fraction:
    """Exact value of an E4M3FN byte, taken from torch's float8 decoder."""
    t = torch.tensor([code & 0xFF], dtype=torch.uint8).view(torch.float8_e4m3fn)
    v = float(t.to(torch.float64).item())
    if v != v:
        raise ValueError("NaN code")
    return Fraction(v)


def e2m1_fraction(nibble: int) -> Fraction:
    """E2M1 from its bit fields: sign bit 3, exponent bits 2-1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (m * 1/2)."""
    s = (nibble >> 3) & 1
    e = (nibble >> 1) & 3
    m = nibble & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


E4M3_POS = [e4m3_fraction(c) for c in range(127)]     # codes 0..126
E2M1_POS = [e2m1_fraction(c) for c in range(8)]       # codes 0..7


def nearest_even(value: Fraction, grid) -> int:
    """Index of the grid value nearest to ``value``; ties go to the even index."""
    best, best_d = None, None
    for i, gv in enumerate(grid):
        d = abs(gv - value)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def round_fp32(value: Fraction) -> Fraction:
    """Round a non-negative rational to the nearest fp32 (ties to even),
    subnormals included."""
    if value == 0:
        return Fraction(0)
    assert value > 0
    e = value.numerator.bit_length() - value.denominator.bit_length()
    if Fraction(2) ** e > value:
        e -= 1
    q = max(e - 23, -149)                 # exponent of the last kept bit
    scaled = value / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * Fraction(2) ** q


def quantize_bruteforce(x: np.ndarray, global_scale=None):
    """Exact-rational NVFP4 quantiser: nearest-by-distance, one rounding each.

    Returns (nibbles [rows, K] int, scale codes [rows, K/16] int, g Fraction).
    """
    rows, cols = x.shape
    vals = [[Fraction(float(v)) for v in row] for row in x]
    if global_scale is None:
        amax = max((abs(v) for row in vals for v in row), default=Fraction(0))
        g = round_fp32(amax / 2688)
    else:
        g = Fraction(float(np.float32(global_scale)))
    nib = np.zeros((rows, cols), dtype=np.int64)
    sc = np.zeros((rows, cols // 16), dtype=np.int64)
    for r in range(rows):
        for b in range(cols // 16):
            blk = vals[r][16 * b:16 * b + 16]
            signs = [1 if np.signbit(float(x[r, 16 * b + i])) else 0 for i in range(16)]
            if g == 0:
                code_s = 0
            else:
                code_s = nearest_even(max(abs(v) for v in blk) / (6 * g), E4M3_POS)
            sc[r, b] = code_s
            S = E4M3_POS[code_s] * g
            for i, v in enumerate(blk):
                mag = 0 if S == 0 else nearest_even(abs(v) / S, E2M1_POS)
                nib[r, 16 * b + i] = (signs[i] << 3) | mag
    return nib, sc, g


def dequant_fraction(nib: np.ndarray, sc: np.ndarray):
    """Exact values E2M1(nib) * E4M3(scale) as nested lists of Fractions."""
    rows, cols = nib.shape
    return [[e2m1_fraction(int(nib[r, k])) * e4m3_fraction(int(sc[r, k // 16]))
             for k in range(cols)] for r in range(rows)]


def unpack_by_hand(q: np.ndarray) -> np.ndarray:
    """Low nibble first: byte j holds elements 2j (bits 0-3) and 2j+1 (4-7)."""
    rows, half = q.shape
    out = np.zeros((rows, 2 * half), dtype=np.int64)
    for r in range(rows):
        for j in range(half):
            out[r, 2 * j] = int(q[r, j]) & 0xF
            out[r, 2 * j + 1] = (int(q[r, j]) >> 4) & 0xF
    return out


def indep_dequant_f64(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Vectorised independent dequantisation (torch float8 + bit fields)."""
    nib = np.concatenate([(q & 0xF)[:, :, None], (q >> 4)[:, :, None]], axis=2)
    nib = nib.reshape(q.shape[0], -1).astype(np.int64)
    e2 = np.array([float(e2m1_fraction(c)) for c in range(16)])[nib]
    sv = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e4m3fn)
    sv = sv.to(torch.float64).numpy()
    return e2 * np.repeat(sv, 16, axis=1)


def e8m0_fraction(code: int) -> Fraction:
    """Exact value of an E8M0 byte, taken from torch's float8_e8m0fnu decoder."""
    t = torch.tensor([code & 0xFF], dtype=torch.uint8).view(torch.float8_e8m0fnu)
    v = float(t.to(torch.float64).item())
    if v != v:
        raise ValueError("NaN code")
    return Fraction(v)


def mx_shared_exponent_bruteforce(amax: Fraction) -> int:
    """Largest E with 2^E <= amax (found by exact comparisons), minus the
    exponent of E2M1's largest value (6 = 1.5 * 2^2), clamped to
    [-127, 127]; -127 for a zero block."""
    if amax == 0:
        return -127
    e = 0
    while Fraction(2) ** e > amax:
        e -= 1
    while Fraction(2) ** (e + 1) <= amax:
        e += 1
    return max(-127, min(127, e - 2))


def mx_quantize_bruteforce(x: np.ndarray):
    """Exact-rational MXFP4 conversion of finite values: per 32-element
    block the shared exponent above, each element the nearest grid value
    E2M1 * 2^E by distance (ties to the even code; beyond 6 * 2^E the
    nearest is 6 * 2^E).  Returns (nibbles [rows, K] int, scale bytes
    [rows, K/32] int)."""
    rows, cols = x.shape
    nib = np.zeros((rows, cols), dtype=np.int64)
    sc = np.zeros((rows, cols // 32), dtype=np.int64)
    for r in range(rows):
        for b in range(cols // 32):
            vals = [Fraction(float(v)) for v in x[r, 32 * b:32 * b + 32]]
            E = mx_shared_exponent_bruteforce(max(abs(v) for v in vals))
            sc[r, b] = E + 127
            grid = [g * Fraction(2) ** E for g in E2M1_POS]
            for i, v in enumerate(vals):
                code = nearest_even(abs(v), grid)
                sign = 1 if np.signbit(x[r, 32 * b + i]) else 0
                nib[r, 32 * b + i] = (sign << 3) | code
    return nib, sc
