"""Pins for the oracle's GEMM, grouped GEMM and tolerance (CPU only).

Operands here are packed by hand (not through the oracle's quantiser) and
expected values come from closed forms or exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import check_gemm, gemm_ref, grouped_gemm_ref, tolerance, ulp_bf16
from tests.indep import (dequant_fraction, e2m1_fraction, e4m3_fraction,
                         indep_dequant_f64, unpack_by_hand)


def _finite_scale_bytes(rng, shape, lo=0x00, hi=0x7E):
    return rng.integers(lo, hi + 1, size=shape).astype(np.uint8)


def _rand_operand(rng, rows, K):
    q = rng.integers(0, 256, size=(rows, K // 2)).astype(np.uint8)
    s = _finite_scale_bytes(rng, (rows, K // 16), 0x20, 0x50)
    return q, s


def _put_nibble(q, r, k, nib):
    """Store nibble at element k of row r: low nibble for even k."""
    j = k // 2
    if k % 2 == 0:
        q[r, j] = (q[r, j] & 0xF0) | nib
    else:
        q[r, j] = (q[r, j] & 0x0F) | (nib << 4)


def test_identity():
    rng = np.random.default_rng(0)
    K = M = 64
    N = 48
    a_q = np.zeros((M, K // 2), dtype=np.uint8)
    for i in range(M):
        _put_nibble(a_q, i, i, 0x2)              # 1.0
    a_s = np.full((M, K // 16), 0x38, dtype=np.uint8)
    b_q, b_s = _rand_operand(rng, N, K)
    gb = np.float32(0.375)
    y, bound = gemm_ref(a_q, a_s, np.float32(1.0), b_q, b_s, gb)
    expect = indep_dequant_f64(b_q, b_s).T * float(gb)
    assert np.array_equal(y, expect)
    assert np.array_equal(bound, np.abs(expect))


@pytest.mark.parametrize("k0", [0, 1, 14, 15, 16, 17, 94, 127])
def test_one_hot_pins_nibble_order_and_scale_index(k0):
    rng = np.random.default_rng(k0)
    M, N, K = 4, 8, 128
    m0 = 2
    a_q = np.zeros((M, K // 2), dtype=np.uint8)
    a_s = np.full((M, K // 16), 0x38, dtype=np.uint8)
    _put_nibble(a_q, m0, k0, 0xB)                 # -1.5
    a_s[m0, k0 // 16] = 0x40                      # 2.0
    b_q, b_s = _rand_operand(rng, N, K)
    ga, gb = np.float32(0.5), np.float32(3.0)
    y, _ = gemm_ref(a_q, a_s, ga, b_q, b_s, gb)
    wd = indep_dequant_f64(b_q, b_s)
    want = np.zeros((M, N))
    want[m0] = -1.5 * 2.0 * wd[:, k0] * 0.5 * 3.0
    assert np.array_equal(y, want)


@pytest.mark.parametrize("cx,sx,cw,sw", [(0x7, 0x7E, 0x7, 0x7E), (0x1, 0x01, 0x9, 0x3C),
                                         (0x5, 0x33, 0xD, 0x47)])
def test_all_equal_closed_form(cx, sx, cw, sw):
    M, N, K = 3, 5, 96
    a_q = np.full((M, K // 2), cx | (cx << 4), dtype=np.uint8)
    a_s = np.full((M, K // 16), sx, dtype=np.uint8)
    b_q = np.full((N, K // 2), cw | (cw << 4), dtype=np.uint8)
    b_s = np.full((N, K // 16), sw, dtype=np.uint8)
    ga, gb = np.float32(1.25), np.float32(0.0625)
    y, _ = gemm_ref(a_q, a_s, ga, b_q, b_s, gb)
    want = (K * Fraction(1.25) * Fraction(0.0625) * e2m1_fraction(cx) * e4m3_fraction(sx)
            * e2m1_fraction(cw) * e4m3_fraction(sw))
    assert np.all(y == float(want))


def test_block_scale_sweep():
    rng = np.random.default_rng(5)
    M, N, K = 2, 3, 256
    a_q = np.full((M, K // 2), 0x22, dtype=np.uint8)     # all 1.0
    b_q = np.full((N, K // 2), 0x22, dtype=np.uint8)
    a_s = _finite_scale_bytes(rng, (M, K // 16), 0x01, 0x7E)
    b_s = _finite_scale_bytes(rng, (N, K // 16), 0x01, 0x7E)
    y, _ = gemm_ref(a_q, a_s, np.float32(1.0), b_q, b_s, np.float32(1.0))
    for m in range(M):
        for n in range(N):
            want = 16 * sum(e4m3_fraction(int(a_s[m, b])) * e4m3_fraction(int(b_s[n, b]))
                            for b in range(K // 16))
            assert y[m, n] == float(want)


@pytest.mark.parametrize("K", [16, 32, 48])
@pytest.mark.parametrize("seed", range(3))
def test_exact_bruteforce_tiny(K, seed):
    rng = np.random.default_rng(1000 * K + seed)
    M, N = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    a_q, a_s = _rand_operand(rng, M, K)
    b_q, b_s = _rand_operand(rng, N, K)
    a_s[:, 0] = _finite_scale_bytes(rng, (M,), 0x00, 0x7E)   # full scale range
    ga, gb = np.float32(rng.random() + 0.1), np.float32(rng.random() * 4)
    y, bound = gemm_ref(a_q, a_s, ga, b_q, b_s, gb)
    xa = dequant_fraction(unpack_by_hand(a_q), a_s)
    wb = dequant_fraction(unpack_by_hand(b_q), b_s)
    alpha = Fraction(float(ga)) * Fraction(float(gb))
    for m in range(M):
        for n in range(N):
            exact = alpha * sum(xa[m][k] * wb[n][k] for k in range(K))
            abs_sum = abs(alpha) * sum(abs(xa[m][k] * wb[n][k]) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= K * Fraction(2) ** -52 * abs_sum
            assert abs(Fraction(float(bound[m, n])) - abs_sum) <= K * Fraction(2) ** -52 * abs_sum


def _simulated_fp32_blocked(a_q, a_s, ga, b_q, b_s, gb):
    """fp32 accumulation of 16-wide block partials, sequential over blocks."""
    xa = indep_dequant_f64(a_q, a_s).astype(np.float32)
    wb = indep_dequant_f64(b_q, b_s).astype(np.float32)
    M, K = xa.shape
    acc = np.zeros((M, wb.shape[0]), dtype=np.float32)
    for b in range(K // 16):
        acc = acc + (xa[:, 16 * b:16 * b + 16] @ wb[:, 16 * b:16 * b + 16].T).astype(np.float32)
    return acc * np.float32(np.float32(ga) * np.float32(gb))


def test_tolerance_accepts_fp32_accumulation_and_rejects_mistakes():
    rng = np.random.default_rng(9)
    M, N, K = 16, 24, 2048
    a_q, a_s = _rand_operand(rng, M, K)
    b_q, b_s = _rand_operand(rng, N, K)
    ga, gb = np.float32(0.01), np.float32(0.02)
    y_ref, bound = gemm_ref(a_q, a_s, ga, b_q, b_s, gb)
    y32 = _simulated_fp32_blocked(a_q, a_s, ga, b_q, b_s, gb)
    ok, worst = check_gemm(y32, y_ref, bound, "f32")
    assert ok and worst < 1 / 16
    yb = torch.from_numpy(y32).to(torch.bfloat16).to(torch.float64).numpy()
    assert check_gemm(yb, y_ref, bound, "bf16")[0]
    assert not check_gemm(yb, y_ref, bound, "f32")[0]     # bf16 needs the ulp term
    # a dropped K-block, a transposed scale, a wrong sign must all fail
    b_drop = b_q.copy()
    b_drop[:, :8] = 0
    y_drop, _ = gemm_ref(a_q, a_s, ga, b_drop, b_s, gb)
    assert not check_gemm(y_drop, y_ref, bound, "f32")[0]
    b_s2 = b_s.copy()
    b_s2[:, [0, 1]] = b_s2[:, [1, 0]]
    y_sw, _ = gemm_ref(a_q, a_s, ga, b_q, b_s2, gb)
    assert not check_gemm(y_sw, y_ref, bound, "f32")[0]
    assert not check_gemm(-y_ref, y_ref, bound, "f32")[0]


def test_ulp_bf16_matches_torch_spacing():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(500) * 10.0 ** rng.integers(-20, 20, size=500)
    vb = torch.from_numpy(v).to(torch.bfloat16)
    # next representable value away from zero: raw pattern + 1 for either sign
    bits = vb.view(torch.int16).to(torch.int32) & 0xFFFF
    nxt = ((bits + 1) & 0xFFFF).to(torch.int32)
    nxt = torch.where(nxt >= 0x8000, nxt - 0x10000, nxt).to(torch.int16).view(torch.bfloat16)
    spacing = (nxt.to(torch.float64) - vb.to(torch.float64)).abs().numpy()
    assert np.array_equal(ulp_bf16(vb.to(torch.float64).numpy()), spacing)
    assert ulp_bf16(np.array([0.0]))[0] == 0.0
    assert ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7


def test_zero_row_requires_exact_zero():
    rng = np.random.default_rng(2)
    a_q, a_s = _rand_operand(rng, 3, 64)
    a_q[1] = 0
    b_q, b_s = _rand_operand(rng, 4, 64)
    y_ref, bound = gemm_ref(a_q, a_s, np.float32(1), b_q, b_s, np.float32(1))
    assert np.all(tolerance(y_ref, bound, "f32")[1] == 0)
    y = y_ref.copy()
    y[1, 2] = 1e-30
    assert not check_gemm(y, y_ref, bound, "f32")[0]


def test_grouped_equals_per_group_concatenation():
    rng = np.random.default_rng(12)
    K, N = 64, 20
    counts = [3, 0, 5, 1, 0, 7]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(off[-1])
    a_q, a_s = _rand_operand(rng, total, K)
    G = len(counts)
    b_q = np.stack([_rand_operand(rng, N, K)[0] for _ in range(G)])
    b_s = np.stack([_rand_operand(rng, N, K)[1] for _ in range(G)])
    b_g = rng.random(G).astype(np.float32)
    ga = np.float32(0.7)
    y, bound = grouped_gemm_ref(off, a_q, a_s, ga, b_q, b_s, b_g)
    assert y.shape == (total, N)
    for e in range(G):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            xa = indep_dequant_f64(a_q[r0:r1], a_s[r0:r1])
            wb = indep_dequant_f64(b_q[e], b_s[e])
            want = xa @ wb.T * (float(ga) * float(b_g[e]))
            np.testing.assert_allclose(y[r0:r1], want, rtol=1e-12, atol=0)
    # permuting the groups permutes the output row blocks
    perm = [5, 2, 0, 3, 1, 4]
    counts_p = [counts[p] for p in perm]
    off_p = np.concatenate([[0], np.cumsum(counts_p)]).astype(np.int32)
    rows_p = np.concatenate([np.arange(off[p], off[p + 1]) for p in perm]).astype(np.int64)
    y_p, _ = grouped_gemm_ref(off_p, a_q[rows_p], a_s[rows_p], ga, b_q[perm], b_s[perm], b_g[perm])
    assert np.array_equal(y_p, y[rows_p])
