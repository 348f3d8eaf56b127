"""GEMM with NVFP4 output (quantisation fused into the epilogue, static
global scale) through the C ABI.

The fused output must be, byte for byte, the oracle's quantisation (with the
same global scale) of the fp32 values the plain GEMM returns for the same
operands: the GEMM's own fp32 result is the input of the encoding, so the
quantised codes are decided in the same precision on both sides.  Those
fp32 values are themselves checked against the fp64 oracle GEMM.  Shapes
cover every kernel of the dispatch: the decode kernel (one and two passes),
the three MFMA tile configurations with ragged edges, and the general kernel.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
from oracle import check_gemm, gemm_ref, pack_nibbles, quantize_ref
from tests.gpu_util import need_gpu, note, np_, to_gpu

pytestmark = pytest.mark.gpu


def _rand_packed(rng, rows, K, lo=0x20, hi=0x48):
    q = rng.integers(0, 256, size=(rows, K // 2)).astype(np.uint8)
    s = rng.integers(lo, hi + 1, size=(rows, K // 16)).astype(np.uint8)
    return q, s


def _fused_case(M, N, K, g_of, seed, check_fp32=True):
    need_gpu()
    rng = np.random.default_rng(seed)
    a = (*_rand_packed(rng, M, K), np.float32(0.37))
    b = (*_rand_packed(rng, N, K), np.float32(0.21))
    ga, gb = to_gpu(*a), to_gpu(*b)
    note(f"gemm nvfp4 out M={M} N={N} K={K}")
    y32 = nv.nvfp4_gemm(ga, gb, out_dtype="f32")
    torch.cuda.synchronize()
    y_np = np_(y32)
    if check_fp32:
        y_ref, bound = gemm_ref(*a, *b)
        ok, worst = check_gemm(y_np, y_ref, bound, "f32")
        assert ok, worst
    g = np.float32(g_of(y_np))
    yg = torch.tensor([float(g)], dtype=torch.float32, device="cuda")
    q, s, _ = nv.nvfp4_gemm_nvfp4_out(ga, gb, yg)
    torch.cuda.synchronize()
    rq, rs, rg = quantize_ref(y_np, global_scale=g)
    assert np.float32(rg) == g
    gq, gs = np_(q), np_(s)
    bad = np.argwhere(gs != rs)
    assert bad.size == 0, f"scale bytes differ at {bad[:5].tolist()}"
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, f"packed bytes differ at {bad[:5].tolist()}"
    # the GPU quantiser with the same static scale agrees as well
    q2, s2, _ = nv.nvfp4_quantize(y32, global_scale=yg)
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, s)


def _data_scale(y):
    """The static scale a calibration pass over this output would give."""
    return np.float32(np.abs(y).max() / np.float32(2688.0))


@pytest.mark.parametrize("M,N,K", [
    (1, 8192, 1024),        # decode, one token
    (16, 4096, 2048),       # decode
    (33, 512, 512),         # decode, three token fragments
    (100, 160, 512),        # decode, two passes
    (300, 384, 1024),       # MFMA 128 x 128 tiles, ragged M
    (520, 16304, 256),      # MFMA 256 x 128 tiles, ragged M and N
    (4136, 4128, 128),      # MFMA 256 x 256 tiles, ragged edges
    (37, 48, 48),           # general kernel (K % 128 != 0)
    (200, 64, 80),          # general kernel, several row tiles
])
def test_fused_output_matches_quantised_fp32(M, N, K):
    _fused_case(M, N, K, _data_scale, seed=M + N + K)


@pytest.mark.parametrize("M,N,K", [(16, 4096, 2048), (520, 16304, 256), (37, 48, 48)])
def test_fused_output_saturates_under_a_small_scale(M, N, K):
    """A static scale 8x too small: large blocks saturate at scale 448 and code 6."""
    _fused_case(M, N, K, lambda y: _data_scale(y) / np.float32(8.0), seed=7 * M + N, check_fp32=False)


@pytest.mark.parametrize("M,N,K", [(16, 4096, 2048), (300, 384, 1024), (37, 48, 48)])
def test_fused_output_zero_and_tiny_scales(M, N, K):
    """g = 0 (scale bytes 0, magnitude codes 0, signs kept) and g below 2^-88
    (the encoder's exact-threshold mode; everything saturates)."""
    _fused_case(M, N, K, lambda y: np.float32(0.0), seed=M, check_fp32=False)
    _fused_case(M, N, K, lambda y: np.float32(2.0 ** -100), seed=M + 1, check_fp32=False)


def _e4m3(c):
    e, m = c >> 3, c & 7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


# E2M1 midpoint m (between two magnitudes) written as hi + lo / 2 with hi, lo
# E2M1 magnitudes, so that m * v = hi * v + lo * (v / 2) for an E4M3 value v
_MID_SPLIT = {0.25: (0.0, 0.5), 0.75: (0.5, 0.5), 1.25: (1.0, 0.5), 1.75: (1.5, 0.5),
              2.5: (2.0, 1.0), 3.5: (3.0, 1.0), 5.0: (4.0, 2.0)}
_E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def _midpoint_operands(M, K):
    """A: M identical rows, nibble 1.0 at K-positions 0 and 16 (blocks 0 and
    1, scale 1.0, g = 1), so y[:, n] = gb * (W[n, 0] + W[n, 16]).  W has 16
    rows per output block j.  Row 16j holds 3.0 x E4M3(k) at position 0 and
    3.0 x E4M3(k + 1) at 16: y = gb * 6 * (the midpoint between codes k and
    k + 1), so under y_g = gb the block's scale quotient is that midpoint
    exactly.  Rows 16j + 1 .. 7 sum to each E2M1 midpoint times E4M3(c), c
    the even one of k, k + 1 (the block's scale code), rows + 8 .. 14 the
    same negated, row 16j + 15 zero."""
    ks = list(range(16, 98))                 # 6 * 2^120 * the midpoint stays finite
    N = 16 * len(ks)
    nib = np.zeros((N, K), np.uint8)
    sc = np.full((N, K // 16), 0x38, np.uint8)
    for j, k in enumerate(ks):
        r = 16 * j
        nib[r, 0], nib[r, 16] = 0x5, 0x5
        sc[r, 0], sc[r, 1] = k, k + 1
        c = k if k % 2 == 0 else k + 1
        for i, m in enumerate(sorted(_MID_SPLIT)):
            hi, lo = _MID_SPLIT[m]
            assert hi * _e4m3(c) + lo * _e4m3(c - 8) == m * _e4m3(c)
            for sign, rr in ((0, r + 1 + i), (8, r + 8 + i)):
                nib[rr, 0] = sign | _E2M1_CODE[hi]
                nib[rr, 16] = sign | _E2M1_CODE[lo]
                sc[rr, 0], sc[rr, 1] = c, c - 8
    a_nib = np.zeros((M, K), np.uint8)
    a_nib[:, 0] = 0x2
    a_nib[:, 16] = 0x2
    a = (pack_nibbles(a_nib), np.full((M, K // 16), 0x38, np.uint8), np.float32(1))
    b = (pack_nibbles(nib), sc, np.float32(2.0 ** 120))
    return a, b


@pytest.mark.parametrize("M,K", [(4, 1024), (40, 256), (256, 128), (4, 48)])
def test_large_output_scale_on_midpoints(M, K):
    """y_g = 2^120 and its fp32 neighbours (the exact-threshold encoder mode):
    outputs exactly on E4M3 scale midpoints and E2M1 element midpoints (and,
    with the neighbouring scales, one ulp of the quotient either side),
    through each kernel of the dispatch (decode through LDS, decode in
    64-row passes, MFMA tiles, general).  Bytes equal the oracle's encoding
    of the fp32 output."""
    need_gpu()
    a, b = _midpoint_operands(M, K)
    ga, gb = to_gpu(*a), to_gpu(*b)
    note(f"gemm nvfp4 out on midpoints M={M} K={K}")
    y32 = nv.nvfp4_gemm(ga, gb, out_dtype="f32")
    torch.cuda.synchronize()
    y_np = np_(y32)
    y_ref, bound = gemm_ref(*a, *b)
    assert np.array_equal(y_np.astype(np.float64), y_ref)      # every output exact
    g0 = np.float32(2.0 ** 120)
    for g in (g0, np.nextafter(g0, np.float32(np.inf)), np.nextafter(g0, np.float32(0))):
        yg = torch.tensor([float(g)], dtype=torch.float32, device="cuda")
        q, s, _ = nv.nvfp4_gemm_nvfp4_out(ga, gb, yg)
        torch.cuda.synchronize()
        rq, rs, _ = quantize_ref(y_np, global_scale=g)
        assert np.array_equal(np_(s), rs), f"scale bytes differ (g = {g})"
        assert np.array_equal(np_(q), rq), f"packed bytes differ (g = {g})"
