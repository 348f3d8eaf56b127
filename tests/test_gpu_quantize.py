"""GPU quantiser vs the oracle: packed nibbles, scale bytes and the global
scale must be identical (the encoding is unique)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from tests.gpu_util import (assert_bytes_equal, need_gpu, note, np_, oracle_global_scale,
                            oracle_quantize)

pytestmark = pytest.mark.gpu


def _check(x_cpu, global_scale=None, ld=None):
    need_gpu()
    x = x_cpu.cuda()
    if ld is not None:                     # strided rows: a view into a wider buffer
        wide = torch.zeros((x.shape[0], ld), dtype=x.dtype, device="cuda")
        wide[:, :x.shape[1]] = x
        x = wide[:, :x_cpu.shape[1]]
    gs = None if global_scale is None else torch.tensor([global_scale], dtype=torch.float32,
                                                        device="cuda")
    note(f"quantize shape={tuple(x.shape)} dtype={x.dtype} ld={x.stride(0)} given={gs is not None}")
    q, s, g = nv.nvfp4_quantize(x, global_scale=gs)
    torch.cuda.synchronize()
    rq, rs, rg = oracle_quantize(x_cpu, global_scale)
    assert_bytes_equal(q, s, g, rq, rs, rg)


def test_tiny_workload_operands():
    x, w = wl.gemm_inputs(0, wl.TINY)
    _check(x)
    _check(w)


@pytest.mark.parametrize("rows,cols,dtype,outliers", [
    (1, 16, "fp32", False), (3, 48, "bf16", False), (17, 512, "bf16", True),
    (300, 1040, "fp32", True), (64, 4096, "bf16", False), (5, 16, "bf16", True),
])
def test_random_shapes(rows, cols, dtype, outliers):
    x = wl.randn((rows, cols), 77 + rows + cols, dtype, outliers)
    _check(x)


def test_strided_rows():
    x = wl.randn((37, 256), 5, "bf16", True)
    _check(x, ld=264)
    x = wl.randn((9, 96), 6, "fp32")
    _check(x, ld=100)


def test_special_values():
    # zero tensor, signed zeros, a constant, midpoint-tied elements under g = 1
    _check(torch.zeros((4, 64)))
    z = torch.zeros((2, 32))
    z[1, 3] = -0.0
    _check(z)
    _check(torch.full((3, 48), -0.7))
    x = torch.zeros((2, 64))
    x[0, 0] = 2688.0                                   # amax 2688 -> g = 1
    x[0, 16] = 6.0                                     # block scale 1.0
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    x[0, 17:24] = mids
    x[0, 24:31] = -mids
    x[1, 0:7] = mids * 6 * 1.0625 / 6                  # other quotients
    x[1, 16] = 6.0 * 1.0625                            # E4M3 tie -> 0x38
    x[1, 32] = 6.0 * 1.1875                            # E4M3 tie -> 0x3A
    x[1, 48] = 6.0 * 2.0 ** -11                        # scale underflows to 0
    _check(x)
    _check(x.to(torch.bfloat16))


def _e4m3_values():
    """The 127 finite non-negative E4M3 values, by code (bit fields)."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


@pytest.mark.parametrize("gmul", [1.0, 1.5, 0.375])
def test_scale_code_tie_sweep(gmul):
    """Block maxima exactly on every E4M3 midpoint (times 6g), and one fp32
    step either side, with g = gmul exactly (first block holds 2688 * gmul)."""
    v = _e4m3_values()
    mids = (v[:-1] + v[1:]) / 2 * 6 * gmul
    vals = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(0))]).astype(np.float32)
    x = np.zeros((len(vals) + 1, 16), dtype=np.float32)
    x[0, 0] = 2688.0 * gmul
    x[1:, 5] = vals
    x[1:, 9] = -vals / 3                     # a second, smaller element per block
    _check(torch.from_numpy(x))


@pytest.mark.parametrize("gmul", [1.0, 1.5])
def test_element_threshold_sweep(gmul):
    """For every non-zero scale code, elements exactly on each E2M1 midpoint
    times the block scale, and one fp32 step either side (g = gmul)."""
    v = _e4m3_values()
    mid2 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = [np.zeros(16, np.float32)]
    rows[0][0] = 2688.0 * gmul
    for c in range(1, 127):
        S = v[c] * gmul
        for side in (0, 1, 2):
            blk = np.zeros(16, np.float32)
            blk[0] = np.float32(6 * S)            # block max 6 S -> scale code c exactly
            t = (mid2 * S).astype(np.float32)
            if side == 1:
                t = np.nextafter(t, np.float32(np.inf))
            elif side == 2:
                t = np.nextafter(t, np.float32(0))
            blk[1:8] = t
            blk[8:15] = -t
            rows.append(blk)
    _check(torch.from_numpy(np.stack(rows)))


@pytest.mark.parametrize("scale", [1e-30, 1e-41, 3e-45])
def test_tiny_magnitudes(scale):
    """Global scales far below the normal range (fp32 subnormal inputs too)."""
    x = (wl.randn((16, 256), 31, "fp32") * scale).to(torch.float32)
    _check(x)


def test_static_global_scale_path():
    x = wl.randn((33, 512), 9, "bf16", True)
    _check(x, global_scale=0.001953125)               # saturates the outliers
    _check(x, global_scale=float(oracle_global_scale(x)))
    _check(x, global_scale=0.0)


def test_linear_workload_activation_full():
    x, _ = wl.gemm_inputs(1, wl.LINEAR)
    _check(x)


def test_large_outlier_workload_sampled_rows():
    need_gpu()
    note("quantize large outlier workload x (16384^2 bf16), sampled rows")
    x_cpu = wl.randn((wl.LARGE.M, wl.LARGE.K), wl.seed_for(4, 0), "bf16", True)
    q, s, g = nv.nvfp4_quantize(x_cpu.cuda())
    torch.cuda.synchronize()
    gref = oracle_global_scale(x_cpu)
    rows = np.sort(np.random.default_rng(0).choice(wl.LARGE.M, 256, replace=False))
    rq, rs, rg = oracle_quantize(x_cpu[torch.from_numpy(rows)], global_scale=gref)
    assert_bytes_equal(q, s, g, rq, rs, gref, rows=rows)


def test_repeat_is_bitwise_identical():
    need_gpu()
    x = wl.randn((512, 2048), 3, "bf16", True).cuda()
    a = nv.nvfp4_quantize(x)
    b = nv.nvfp4_quantize(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


_BIG = float(np.float32(2.0 ** 116))
_LARGE_G = [2.0 ** 120, 1e37, 3e38, _BIG, float(np.nextafter(np.float32(_BIG), np.float32(0)))]


@pytest.mark.parametrize("g", _LARGE_G)
def test_large_static_scale_scale_code_ties(g):
    """Static global scales at and above 2^116, where 1 / 6g and
    1 / (E4M3(s) g) leave the normal fp32 range: block maxima on every E4M3
    midpoint times 6g that fp32 can hold, and one fp32 step either side."""
    v = _e4m3_values()
    mids = (v[:-1] + v[1:]) / 2 * 6 * np.float64(np.float32(g))
    mids = mids[mids < np.finfo(np.float32).max / 2]
    m32 = mids.astype(np.float32)
    vals = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)),
                           np.nextafter(m32, np.float32(0))])
    vals = vals[np.isfinite(vals) & (vals > 0)]
    x = np.zeros((len(vals), 16), dtype=np.float32)
    x[:, 5] = vals
    x[:, 9] = -vals / 3
    x[:, 12] = vals / 7
    _check(torch.from_numpy(x), global_scale=g)


@pytest.mark.parametrize("g", _LARGE_G)
def test_large_static_scale_element_thresholds(g):
    """For every scale code whose block fits fp32 under static scale g: a
    block maximum of 6 E4M3(c) g and elements on each E2M1 midpoint times
    E4M3(c) g, and one fp32 step either side."""
    v = _e4m3_values()
    gd = np.float64(np.float32(g))
    mid2 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for c in range(1, 127):
        S = v[c] * gd
        if 6 * S >= np.finfo(np.float32).max / 2:
            break
        for side in (0, 1, 2):
            blk = np.zeros(16, np.float32)
            blk[0] = np.float32(6 * S)
            t = (mid2 * S).astype(np.float32)
            if side == 1:
                t = np.nextafter(t, np.float32(np.inf))
            elif side == 2:
                t = np.nextafter(t, np.float32(0))
            blk[1:8] = t
            blk[8:15] = -t
            rows.append(blk)
    _check(torch.from_numpy(np.stack(rows)), global_scale=g)


@pytest.mark.parametrize("g", [1e37, 3e38])
def test_large_static_scale_random(g):
    """Random data, outliers included, under huge static scales (most scale
    codes subnormal or zero)."""
    x = wl.randn((64, 512), 41, "fp32", True) * 1e36
    _check(x, global_scale=g)
    _check(x.to(torch.bfloat16), global_scale=g)
