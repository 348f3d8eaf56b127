"""Pins for the oracle's quantiser (CPU only).

Midpoint cases are built so that the exact quotients are known: a block whose
amax is 6*t under a global scale of exactly 1 has the E4M3 quotient t; a block
with amax 6 then has scale 1.0 and each element's E2M1 quotient is the element
itself.
"""
import numpy as np
import pytest
import torch

from oracle import dequantize_ref, e4m3_decode, quantize_ref, unpack_nibbles
from tests.indep import quantize_bruteforce, round_fp32

from fractions import Fraction


def _scale_code(t, via_amax_2688=False):
    """Scale byte of a block with amax 6t, under g = 1."""
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, 0] = 6.0 * t
    if via_amax_2688:
        blk[0, 16] = 2688.0          # separate block: amax_t = 2688 -> g = 1
        q, s, g = quantize_ref(blk)
        assert g == np.float32(1.0)
    else:
        q, s, g = quantize_ref(blk, global_scale=1.0)
    return int(s[0, 0])


@pytest.mark.parametrize("t,code", [
    (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A), (1.9375, 0x40),
    (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (448.0, 0x7E),
    (460.0, 0x7E), (500.0, 0x7E), (3.0 * 2.0 ** -10, 0x02), (0.0, 0x00),
])
def test_e4m3_scale_rounding_pins(t, code):
    assert _scale_code(t) == code
    if 6.0 * t <= 2688.0:
        assert _scale_code(t, via_amax_2688=True) == code


def test_e4m3_scale_rounding_matches_torch_rne_below_464():
    # t with <= 21 significant bits: 6t and t are exact fp32, so torch's fp32
    # -> float8_e4m3fn cast (round to nearest even) sees the exact quotient.
    rng = np.random.default_rng(7)
    mant = rng.integers(1 << 10, 1 << 21, size=400)
    expo = rng.integers(-32, 9, size=400)
    ts = np.ldexp(mant.astype(np.float64) / (1 << 21), expo).astype(np.float32)
    ts = ts[ts < 464.0]
    # every E4M3 midpoint, where ties decide
    pos = e4m3_decode(np.arange(127))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    ts = np.concatenate([ts, mids, pos[1:].astype(np.float32)])
    for t in ts:
        want = int(torch.tensor([float(t)], dtype=torch.float32)
                   .to(torch.float8_e4m3fn).view(torch.uint8).item())
        assert _scale_code(float(t)) == want, t


MID_CASES = [  # (element value with S = 1, expected magnitude code)
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (0.25 + 2 ** -20, 1), (0.25 - 2 ** -20, 0),
    (0.75 - 2 ** -20, 1), (0.75 + 2 ** -20, 2),
    (1.25 - 2 ** -20, 2), (1.25 + 2 ** -20, 3),
    (1.75 - 2 ** -20, 3), (1.75 + 2 ** -20, 4),
    (2.5 - 2 ** -20, 4), (2.5 + 2 ** -20, 5),
    (3.5 - 2 ** -20, 5), (3.5 + 2 ** -20, 6),
    (5.0 - 2 ** -20, 6), (5.0 + 2 ** -20, 7),
    (6.0, 7), (0.5, 1), (3.0, 5), (0.0, 0),
]


@pytest.mark.parametrize("v,code", MID_CASES)
def test_e2m1_element_rounding_pins(v, code):
    blk = np.zeros((1, 16), dtype=np.float32)
    blk[0, 0] = 6.0                    # block amax 6 -> scale 1.0 under g = 1
    blk[0, 1] = v
    blk[0, 2] = -v
    q, s, g = quantize_ref(blk, global_scale=1.0)
    assert s[0, 0] == 0x38
    nib = unpack_nibbles(q)[0]
    assert nib[0] == 0x7
    assert nib[1] == code
    assert nib[2] == (0x8 | code)


def test_saturation_of_elements_above_six():
    # 6.375 arises when the block scale rounds down: amax_b = 6 * 1.0625*... ;
    # here built directly with a block scale of 1 and an element 6.25
    blk = np.zeros((1, 16), dtype=np.float32)
    blk[0, 0] = 6.25                   # quotient 6.25/6 -> E4M3 1.0 (0x38)
    q, s, g = quantize_ref(blk, global_scale=1.0)
    assert s[0, 0] == 0x38
    assert unpack_nibbles(q)[0, 0] == 0x7


def test_signed_zero_and_tiny_negatives():
    blk = np.zeros((1, 16), dtype=np.float32)
    blk[0, 0] = 6.0
    blk[0, 1] = -0.0
    blk[0, 2] = -1e-9
    blk[0, 3] = 1e-9
    q, s, g = quantize_ref(blk, global_scale=1.0)
    nib = unpack_nibbles(q)[0]
    assert list(nib[1:4]) == [0x8, 0x8, 0x0]


def test_constant_tensor_closed_form():
    for c in (1.0, 3.14159, 1e-20, 1e20, 0.7):
        x = np.full((3, 64), c, dtype=np.float32)
        q, s, g = quantize_ref(x)
        assert np.all(s == 0x7E)
        assert np.all(q == 0x77)
        q, s, g = quantize_ref(-x)
        assert np.all(s == 0x7E)
        assert np.all(q == 0xFF)


def test_zero_tensor():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 5] = -0.0
    q, s, g = quantize_ref(x)
    assert g == 0.0
    assert np.all(s == 0)
    nib = unpack_nibbles(q)
    assert nib[1, 5] == 0x8
    nib[1, 5] = 0
    assert np.all(nib == 0)


def test_zero_block_inside_nonzero_tensor():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 20] = 5.0
    q, s, g = quantize_ref(x)
    assert s[0, 0] == 0 and s[0, 1] == 0x7E
    assert np.all(unpack_nibbles(q)[0, :16] == 0)


def test_underflowing_block_scale_zeroes_block():
    # amax_b / (6 g) below the smallest E4M3 half-step -> scale 0 -> magnitudes 0
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 2688.0                   # g = 1
    x[0, 16] = 6.0 * 2.0 ** -11        # quotient 2^-11 < 2^-10 -> scale 0
    x[0, 17] = -6.0 * 2.0 ** -11
    q, s, g = quantize_ref(x)
    assert s[0, 1] == 0
    nib = unpack_nibbles(q)[0]
    assert nib[16] == 0 and nib[17] == 0x8


def test_global_scale_is_ieee_fp32_division():
    rng = np.random.default_rng(3)
    for _ in range(200):
        a = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-30, 30))
        x = np.array([[a] + [0.0] * 15], dtype=np.float32)
        q, s, g = quantize_ref(x)
        assert Fraction(float(g)) == round_fp32(Fraction(float(a)) / 2688)


def _assert_matches_bruteforce(x, global_scale=None):
    q, s, g = quantize_ref(x, global_scale=global_scale)
    nib_b, sc_b, g_b = quantize_bruteforce(x, global_scale=global_scale)
    assert Fraction(float(g)) == g_b
    assert np.array_equal(s.astype(np.int64), sc_b)
    assert np.array_equal(unpack_nibbles(q).astype(np.int64), nib_b)


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_random_normal(seed):
    rng = np.random.default_rng(seed)
    shape = [(3, 32), (2, 48), (1, 16), (4, 16), (2, 64), (3, 16)][seed]
    x = rng.standard_normal(shape).astype(np.float32)
    if seed % 2:
        x *= np.where(rng.random(shape) < 0.1, 50.0, 1.0).astype(np.float32)
    _assert_matches_bruteforce(x)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    _assert_matches_bruteforce(xb)


@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_tie_rich(seed):
    # elements placed exactly on E2M1 midpoints of random E4M3 block scales,
    # under power-of-two global scales, plus random scale-code midpoints
    rng = np.random.default_rng(100 + seed)
    pos = e4m3_decode(np.arange(127))
    g = 2.0 ** int(rng.integers(-4, 5))
    rows = []
    for r in range(3):
        row = []
        for b in range(2):
            c = int(rng.integers(1, 127))
            S = pos[c] * g
            mids = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], size=15)
            sgn = rng.choice([-1.0, 1.0], size=15)
            blk = [6.0 * S] + list(sgn * mids * S)
            row += blk
        rows.append(row)
    x = np.array(rows, dtype=np.float32)
    _assert_matches_bruteforce(x, global_scale=g)
    # E4M3 midpoints as block quotients: amax_b = 6 * g * mid(c)
    mids = (pos[:-1] + pos[1:]) / 2
    x2 = np.zeros((2, 64), dtype=np.float32)
    picks = rng.choice(len(mids), size=8, replace=False)
    for i, c in enumerate(picks):
        x2[i // 4, 16 * (i % 4)] = np.float32(6.0 * g * mids[c])
        x2[i // 4, 16 * (i % 4) + 1] = np.float32(-3.0 * g * mids[c])
    _assert_matches_bruteforce(x2, global_scale=g)


def test_dequant_error_bound():
    # every element lies within half an E2M1 step (times the block scale) of
    # its decoded value, except saturated ones (|v| <= 6.375 S)
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 256)) * np.where(rng.random((8, 256)) < 0.02, 50, 1)).astype(np.float32)
    q, s, g = quantize_ref(x)
    d = dequantize_ref(q, s) * float(g)
    S = np.repeat(e4m3_decode(s), 16, axis=1) * float(g)
    err = np.abs(d - x.astype(np.float64))
    half_step = np.where(np.abs(x) < 2 * S, 0.25, np.where(np.abs(x) < 4 * S, 0.5, 1.0)) * S
    assert np.all(err <= half_step + 1e-30)
