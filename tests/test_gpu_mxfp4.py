"""GPU MXFP4 variant vs the oracle, through the C ABI: the conversion bit for
bit, the GEMM within the stated tolerance (matrix-core kernel and general
kernel), at small sizes over several tiles with ragged edges and at the
linear workload's full size on sampled rows and outputs."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from oracle import (check_gemm, mxfp4_dequantize_ref, mxfp4_gemm_ref, mxfp4_quantize_ref,
                    pack_nibbles)
from tests.gpu_util import need_gpu, note, np_

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _t(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(DEV)


def _quantize_check(x_cpu: torch.Tensor, x_dev: torch.Tensor | None = None):
    q, s = nv.nvfp4_mxfp4_quantize(x_cpu.to(DEV) if x_dev is None else x_dev)
    torch.cuda.synchronize()
    rq, rs = mxfp4_quantize_ref(x_cpu.float().numpy())
    gq, gs = np_(q), np_(s)
    assert np.array_equal(gs, rs), np.argwhere(gs != rs)[:5]
    assert np.array_equal(gq, rq), np.argwhere(gq != rq)[:5]
    return q, s


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (130, 512), (257, 1024)])
def test_quantize_bit_exact(dtype, rows, cols):
    x = wl.randn((rows, cols), rows * 31 + cols, dtype)
    # blocks over a wide range of magnitudes
    x = x * torch.exp2(torch.randint(-40, 40, (rows, 1)).to(x.dtype))
    note(f"mxfp4 quantize {dtype} {rows}x{cols}")
    _quantize_check(x)


def test_quantize_special_blocks():
    """Zero, signed-zero, subnormal-only, near-fp32-max, tie-rich, saturating
    and non-finite blocks, fp32 input."""
    rng = np.random.default_rng(7)
    x = np.zeros((8, 64), np.float32)
    x[1, :32] = -0.0
    x[2, :] = np.float32(2.0 ** -149) * rng.integers(1, 100, 64)
    x[3, :] = np.float32(3.0e38) * rng.uniform(-1, 1, 64).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x[4, :] = np.concatenate([rng.choice(mids, 31), [7.5], rng.choice(mids, 31) * -4, [30.0]])
    x[5, :] = np.linspace(-8, 8, 64, dtype=np.float32)          # amax 8: E = 1
    x[6, 10] = np.inf
    x[6, 40] = 1.0
    x[7, 33] = np.nan
    x[7, 0] = -3.0
    note("mxfp4 quantize special blocks")
    q, s = nv.nvfp4_mxfp4_quantize(_t(x))
    torch.cuda.synchronize()
    rq, rs = mxfp4_quantize_ref(x)
    assert np.array_equal(np_(s), rs) and np.array_equal(np_(q), rq)


def test_quantize_strided_rows():
    x_full = wl.randn((64, 256 + 64), 5, "bf16")
    x_view = x_full.to(DEV)[:, 32:32 + 256]
    note("mxfp4 quantize strided rows")
    _quantize_check(x_full[:, 32:32 + 256].contiguous(), x_view)


def _rand_mx(rng, rows, K, lo=112, hi=142):
    q = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    s = rng.integers(lo, hi, (rows, K // 32)).astype(np.uint8)
    return q, s


@pytest.mark.parametrize("M,N,K", [
    (64, 64, 128), (128, 256, 512), (200, 72, 384), (1, 300, 256), (300, 33, 1024),
    (256, 512, 256), (96, 40, 96), (17, 9, 32), (5, 130, 160),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_against_oracle(M, N, K, out):
    """K % 128 == 0 runs the matrix-core kernel (tiles 64..256, ragged M and
    N); K = 96, 32, 160 the general kernel."""
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    aq, as_ = _rand_mx(rng, M, K)
    bq, bs = _rand_mx(rng, N, K)
    note(f"mxfp4 gemm {M}x{N}x{K} {out}")
    y = nv.nvfp4_mxfp4_gemm((_t(aq), _t(as_)), (_t(bq), _t(bs)), out)
    torch.cuda.synchronize()
    y_ref, bound = mxfp4_gemm_ref(aq, as_, bq, bs)
    ok, worst = check_gemm(np_(y), y_ref, bound, out)
    assert ok, worst


@pytest.mark.parametrize("M,N,K", [(4096, 1024, 512), (4096, 2048, 256), (4000, 4000, 256),
                                   (4096, 4096, 128)])
def test_gemm_large_tiles(M, N, K):
    """Shapes that reach the 128 x 128, 256 x 128 and 256 x 256 tile
    configurations (ragged edges at 4000; K = 128 is a single stage, so
    every refill is a padding reload); checked on sampled rows."""
    rng = np.random.default_rng(M + N + K)
    aq, as_ = _rand_mx(rng, M, K)
    bq, bs = _rand_mx(rng, N, K)
    note(f"mxfp4 gemm {M}x{N}x{K} (large tiles)")
    y = nv.nvfp4_mxfp4_gemm((_t(aq), _t(as_)), (_t(bq), _t(bs)), "f32")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 60, replace=False)]))
    y_ref, bound = mxfp4_gemm_ref(aq[rows], as_[rows], bq, bs)
    ok, worst = check_gemm(np_(y)[rows], y_ref, bound, "f32")
    assert ok, worst


def test_exhaustive_dequant_identity():
    """One-hot A rows (value 1: code 2 under scale byte 127) read every
    column of B, whose rows hold every nibble under scale bytes 2..252 (the
    range whose values are normal fp32): y is B's values, bit for bit, on the
    matrix-core kernel (K = 512)."""
    K = 512
    scales = np.arange(2, 253, dtype=np.uint8)
    n_rows = int(np.ceil(len(scales) / (K // 32)))
    sb = np.resize(scales, (n_rows, K // 32)).astype(np.uint8)
    rng = np.random.default_rng(3)
    nib = np.stack([np.concatenate([rng.permutation(16), rng.permutation(16)]) for _ in range(n_rows * K // 32)])
    bq = pack_nibbles(nib.reshape(n_rows, K))
    eye = np.zeros((K, K), np.uint8)
    eye[np.arange(K), np.arange(K)] = 2
    aq = pack_nibbles(eye)
    as_ = np.full((K, K // 32), 127, np.uint8)
    note("mxfp4 exhaustive dequant identity")
    y = nv.nvfp4_mxfp4_gemm((_t(aq), _t(as_)), (_t(bq), _t(sb)), "f32")
    torch.cuda.synchronize()
    want = mxfp4_dequantize_ref(bq, sb).T.astype(np.float32)
    assert np.array_equal(np_(y), want)


def test_nan_scale_gives_nan():
    K = 256
    rng = np.random.default_rng(4)
    aq, as_ = _rand_mx(rng, 64, K)
    bq, bs = _rand_mx(rng, 64, K)
    as_[5, 3] = 255
    note("mxfp4 gemm NaN scale")
    y = np_(nv.nvfp4_mxfp4_gemm((_t(aq), _t(as_)), (_t(bq), _t(bs)), "f32"))
    assert np.all(np.isnan(y[5])) and not np.any(np.isnan(np.delete(y, 5, axis=0)))


def test_linear_workload_full_size():
    """x [4096, 8192], W [8192, 8192] bf16 N(0,1), the shapes the bench times:
    the conversion bit-exact on sampled rows of both, the GEMM (256 x 256
    tiles) on sampled outputs."""
    cfg = wl.LINEAR
    x = wl.randn((cfg.M, cfg.K), wl.seed_for(1, 0), "bf16", device=DEV)
    w = wl.randn((cfg.N, cfg.K), wl.seed_for(1, 1), "bf16", device=DEV)
    note("mxfp4 linear workload: quantize x and W")
    xq = nv.nvfp4_mxfp4_quantize(x)
    wq = nv.nvfp4_mxfp4_quantize(w)
    note("mxfp4 linear workload: gemm")
    y = nv.nvfp4_mxfp4_gemm(xq, wq, "bf16")
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    xr = np.unique(np.concatenate([[0, cfg.M - 1], rng.choice(cfg.M, 14, replace=False)]))
    wr = np.unique(np.concatenate([[0, cfg.N - 1], rng.choice(cfg.N, 30, replace=False)]))
    ti = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    rxq, rxs = mxfp4_quantize_ref(x.index_select(0, ti(xr)).float().cpu().numpy())
    rwq, rws = mxfp4_quantize_ref(w.index_select(0, ti(wr)).float().cpu().numpy())
    assert np.array_equal(np_(xq[0])[xr], rxq) and np.array_equal(np_(xq[1])[xr], rxs)
    assert np.array_equal(np_(wq[0])[wr], rwq) and np.array_equal(np_(wq[1])[wr], rws)
    y_ref, bound = mxfp4_gemm_ref(rxq, rxs, rwq, rws)
    ok, worst = check_gemm(np_(y)[np.ix_(xr, wr)], y_ref, bound, "bf16")
    assert ok, worst
