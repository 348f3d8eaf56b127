"""Pins of the MXFP4 oracle (oracle/mxfp4_ref.py) against facts that do not
come from it: torch's E8M0 decoder, exact rational brute force of the
conversion (tests/indep.py), bit-level closed forms and exact rational GEMMs.
The conversion rule itself is the microscaling definition restated in the
oracle's header; no page defines it, so these pins fix the mathematics, not
parity with the pages."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (check_gemm, e8m0_decode, mxfp4_dequantize_ref, mxfp4_gemm_ref,
                    mxfp4_quantize_ref, pack_nibbles, unpack_nibbles)
from oracle.mxfp4_ref import shared_exponent
from tests.indep import (E2M1_POS, e2m1_fraction, e8m0_fraction, mx_quantize_bruteforce,
                         mx_shared_exponent_bruteforce)


def test_e8m0_decode_matches_torch():
    codes = np.arange(255)
    got = e8m0_decode(codes)
    for c in codes:
        assert Fraction(float(got[c])) == e8m0_fraction(int(c))
    assert np.isnan(e8m0_decode([255]))[0]


@pytest.mark.parametrize("v", [1.0, 3.99, 4.0, 5.9, 6.0, 7.99, 8.0, 0.5, 2.0 ** -126, 2.0 ** -149,
                               3 * 2.0 ** -140, 2.0 ** 127, 3.4e38, 1e-30, 448.0, 0.0])
def test_shared_exponent_against_exact_search(v):
    v32 = float(np.float32(v))
    assert int(shared_exponent(v32)) == mx_shared_exponent_bruteforce(Fraction(v32))


def test_shared_exponent_random_fp32():
    rng = np.random.default_rng(1)
    bits = rng.integers(1, 0x7F800000, size=2000, dtype=np.int64).astype(np.uint32)
    vals = bits.view(np.float32).astype(np.float64)
    got = shared_exponent(vals)
    for v, e in zip(vals, got):
        assert int(e) == mx_shared_exponent_bruteforce(Fraction(float(v)))


def _check_bruteforce(x):
    q, s = mxfp4_quantize_ref(x)
    nib_ref, sc_ref = mx_quantize_bruteforce(x)
    assert np.array_equal(unpack_nibbles(q).astype(np.int64), nib_ref)
    assert np.array_equal(s.astype(np.int64), sc_ref)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_conversion_bruteforce_random(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 96)) * np.exp(rng.normal(0, 3, (3, 1)))).astype(np.float32)
    _check_bruteforce(x)


def test_conversion_bruteforce_ties_and_saturation():
    """Every E2M1 midpoint times 2^E, exact grid values and values between
    6 and 8 times 2^E (saturating), with the block maximum fixing E."""
    rng = np.random.default_rng(5)
    rows = []
    for E in (-3, 0, 4):
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        grid = [0.5, 1, 1.5, 2, 3, 4, 6]
        vals = mids + grid + [6.5, 7.0, 7.75, -5.0, -0.25, -0.75, -7.9, 0.0, -0.0]
        vals = vals + list(rng.choice(mids, 32 - len(vals)))
        block = np.array(vals[:31] + [7.99], dtype=np.float64) * 2.0 ** E  # amax in [4, 8)
        rows.append(block.astype(np.float32))
    _check_bruteforce(np.stack(rows))


def test_zero_block_and_extremes():
    x = np.zeros((3, 64), np.float32)
    x[0, 32:] = -0.0
    x[1, :32] = 2.0 ** -149            # smallest subnormal: E clamps to -127
    x[1, 32:] = np.float32(3.4e38)     # E = 125
    x[2, 5] = -1.0
    q, s = mxfp4_quantize_ref(x)
    nib = unpack_nibbles(q)
    assert s[0, 0] == 0 and np.all(nib[0, :32] == 0)
    assert s[0, 1] == 0 and np.all(nib[0, 32:] == 8)          # sign of -0.0 kept
    assert s[1, 0] == 0 and np.all(nib[1, :32] == 0)          # 2^-149 / 2^-127 rounds to 0
    assert s[1, 1] == 127 + 125 and np.all(nib[1, 32:] == 7)  # 3.4e38 / 2^125 ~ 7.99 -> 6
    assert s[2, 0] == 127 - 2 and nib[2, 5] == 0xE            # -1.0 / 2^-2 = -4: sign | code 6
    _check_bruteforce(x)


def test_non_finite_block():
    x = np.ones((1, 64), np.float32)
    x[0, 3] = np.inf
    x[0, 40] = np.nan
    q, s = mxfp4_quantize_ref(x)
    assert s[0, 0] == 255 and s[0, 1] == 255 and np.all(q == 0)


def test_dequantize_bit_fields():
    """Every nibble under a few scale bytes equals E2M1 (bit fields) * 2^(b-127)."""
    nib = np.tile(np.arange(16, dtype=np.uint8), (4, 2))          # [4, 32]
    s = np.array([[0], [100], [127], [254]], np.uint8)
    v = mxfp4_dequantize_ref(pack_nibbles(nib), s)
    for r in range(4):
        for k in range(32):
            assert Fraction(float(v[r, k])) == e2m1_fraction(int(nib[r, k])) * e8m0_fraction(int(s[r, 0]))


@pytest.mark.parametrize("K,seed", [(32, 0), (64, 1), (128, 2)])
def test_gemm_exact_bruteforce_tiny(K, seed):
    rng = np.random.default_rng(seed)
    M, N = 3, 4
    qa = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    y, bound = mxfp4_gemm_ref(qa, sa, qb, sb)
    na, nb = unpack_nibbles(qa), unpack_nibbles(qb)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            acc_abs = Fraction(0)
            for k in range(K):
                t = (e2m1_fraction(int(na[m, k])) * e8m0_fraction(int(sa[m, k // 32]))
                     * e2m1_fraction(int(nb[n, k])) * e8m0_fraction(int(sb[n, k // 32])))
                acc += t
                acc_abs += abs(t)
            assert Fraction(float(y[m, n])) == acc     # exact in fp64 at these sizes
            assert Fraction(float(bound[m, n])) == acc_abs


def test_gemm_one_hot_reads_weight_values():
    """A one-hot row of A (value 1 = code 2 under scale 127) at column k
    reads column k of B's dequantised rows: pins nibble order and the
    32-element scale index."""
    K, N = 64, 3
    rng = np.random.default_rng(9)
    qb = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sb = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    wb = mxfp4_dequantize_ref(qb, sb)
    for k in (0, 1, 31, 32, 33, 63):
        nib = np.zeros((1, K), np.uint8)
        nib[0, k] = 2
        y, _ = mxfp4_gemm_ref(pack_nibbles(nib), np.full((1, 2), 127, np.uint8), qb, sb)
        assert np.array_equal(y[0], wb[:, k])
        b = k // 32
        assert wb[0, k] == float(E2M1_POS[int(unpack_nibbles(qb)[0, k]) & 7]) * \
            (-1 if unpack_nibbles(qb)[0, k] & 8 else 1) * 2.0 ** (int(sb[0, b]) - 127)


def test_round_trip_is_within_half_a_grid_step():
    """Dequantised conversion of N(0,1) data: every element within half a
    grid step of the input (the step at its magnitude), or saturated."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q, s = mxfp4_quantize_ref(x)
    v = mxfp4_dequantize_ref(q, s)
    scale = np.repeat(e8m0_decode(s), 32, axis=1)
    err = np.abs(v - x) / scale
    sat = np.abs(x) / scale > 6
    assert np.all(err[~sat] <= 1.0 + 1e-12)      # largest step (4 -> 6) is 2
    assert np.all(np.abs(v[sat]) == 6 * scale[sat])


def test_tolerance_applies_to_mx_products():
    rng = np.random.default_rng(4)
    qa = rng.integers(0, 256, (4, 64)).astype(np.uint8)
    qb = rng.integers(0, 256, (5, 64)).astype(np.uint8)
    sa = rng.integers(120, 134, (4, 4)).astype(np.uint8)
    sb = rng.integers(120, 134, (5, 4)).astype(np.uint8)
    y, bound = mxfp4_gemm_ref(qa, sa, qb, sb)
    ok, _ = check_gemm(y.astype(np.float32), y, bound, "f32")
    assert ok
    ok, _ = check_gemm(y * (1 + 1e-3) + 1e-3, y, bound, "f32")
    assert not ok
    torch.manual_seed(0)
