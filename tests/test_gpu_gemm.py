"""GPU GEMM vs the oracle, through the C ABI.

Operands are quantised by the oracle on the CPU and uploaded, so the GEMM is
checked independently of the GPU quantiser (whose bytes are compared to the
same oracle output where the GPU quantiser is used).  Tolerance: |y - y_ref|
<= 1e-5 * sum_k |x_k w_k| per element, plus one bf16 ulp for bf16 output.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from oracle import check_gemm, dequantize_ref, e4m3_decode, gemm_ref, pack_nibbles
from tests.gpu_util import (assert_bytes_equal, need_gpu, note, np_, oracle_global_scale,
                            oracle_quantize, to_gpu)

pytestmark = pytest.mark.gpu


def _gemm(a, b, out):
    y = nv.nvfp4_gemm(a, b, out_dtype=out)
    torch.cuda.synchronize()
    return y


def _parity(x_cpu, w_cpu, out="f32", tag=""):
    need_gpu()
    ra = oracle_quantize(x_cpu)
    rb = oracle_quantize(w_cpu)
    note(f"gemm {tag} M={x_cpu.shape[0]} N={w_cpu.shape[0]} K={x_cpu.shape[1]} out={out}")
    y = _gemm(to_gpu(*ra), to_gpu(*rb), out)
    y_ref, bound = gemm_ref(*ra, *rb)
    ok, worst = check_gemm(np_(y), y_ref, bound, out)
    assert ok, f"{tag}: worst |err|/tol = {worst}"
    return y, ra, rb


def _rand_packed(rng, rows, K, lo=0x20, hi=0x50):
    q = rng.integers(0, 256, size=(rows, K // 2)).astype(np.uint8)
    s = rng.integers(lo, hi + 1, size=(rows, K // 16)).astype(np.uint8)
    return q, s


def test_tiny_workload():
    x, w = wl.gemm_inputs(0, wl.TINY)
    y, ra, rb = _parity(x, w, "f32", "tiny")
    # the GPU quantiser produces the same operands
    for t, ref in ((x, ra), (w, rb)):
        assert_bytes_equal(*nv.nvfp4_quantize(t.cuda()), *ref)


@pytest.mark.parametrize("M,K", [(128, 128), (16, 128), (1, 128), (256, 256), (32, 256),
                                 (1, 256), (20, 256)])
def test_exhaustive_dequant_identity(M, K):
    """A = first M rows of I_K (nibble 1.0, scale 1.0, g = 1); W [4096/K, K]
    holds every nibble under every finite scale byte, so y = W_dq^T exactly
    (K = 128 runs the tile kernel, K = 256 with M <= 32 the skinny kernel)."""
    need_gpu()
    N = 4096 // K
    nib = np.zeros((M, K), dtype=np.uint8)
    for i in range(M):
        nib[i, i] = 0x2
    a = (pack_nibbles(nib), np.full((M, K // 16), 0x38, np.uint8), np.float32(1))
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x3F, 0xBF                 # NaN codes replaced
    rng = np.random.default_rng(0)
    wn = np.zeros((N, K), dtype=np.uint8)
    for blk in range(N * K // 16):
        r, c = divmod(blk, K // 16)
        wn[r, 16 * c:16 * c + 16] = rng.permutation(16)
    b = (pack_nibbles(wn), codes.reshape(N, K // 16), np.float32(1))
    note(f"exhaustive dequant M={M}")
    y = np_(_gemm(to_gpu(*a), to_gpu(*b), "f32"))
    y_ref, _ = gemm_ref(*a, *b)
    assert np.array_equal(y, y_ref.astype(np.float32))


@pytest.mark.parametrize("N", [4096, 2048])
def test_exhaustive_dequant_identity_wide_tiles(N):
    """A = I_4096 in FP4 (nibble 1.0, scale 1.0, g = 1) against W [N, 4096]
    whose blocks each hold all 16 nibbles, with every finite scale byte
    repeated across the blocks: y = W_dq^T exactly.  The tile counts select
    the 256 x 256 (N = 4096) and 256 x 128 (N = 2048) configurations."""
    need_gpu()
    K = M = 4096
    nib = np.zeros((M, K), dtype=np.uint8)
    nib[np.arange(M), np.arange(K)] = 0x2
    a = (pack_nibbles(nib), np.full((M, K // 16), 0x38, np.uint8), np.float32(1))
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x3F, 0xBF                 # NaN codes replaced
    rng = np.random.default_rng(N)
    nblk = N * K // 16
    perm = np.argsort(rng.random((nblk, 16)), axis=1).astype(np.uint8)   # a permutation per block
    wn = perm.reshape(N, K)
    ws = np.resize(np.roll(codes, N // 64), nblk).reshape(N, K // 16)
    b = (pack_nibbles(wn), ws, np.float32(1))
    note(f"exhaustive dequant, wide tiles, N={N}")
    y = np_(_gemm(to_gpu(*a), to_gpu(*b), "f32"))
    assert np.array_equal(y, dequantize_ref(b[0], b[1]).T.astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(520, 16300, 128), (512, 16384, 256), (384, 8000, 256),
                                   (256, 8192, 512), (200, 8100, 384),
                                   (130, 5000, 384), (100, 8192, 256), (70, 8150, 384)])
def test_mid_m_tile_configs(M, N, K):
    """Shapes whose tile counts pick each MFMA tile configuration, ragged M
    and N included.  The first two pick 256 x 128, the third 128 x 128.
    The next two pick 128 x 64 (fewer than 256 tiles of 128 x 128, at most
    256 of 128 x 64, or more than 256 of 64 x 64).  The last three pick
    64 x 64.  Of those, (100, 8192) has more than 96 rows and 64 x 64 tiles
    that fill the chip, so the MFMA kernel takes it over from the decode
    kernel's two passes; (70, 8150) gets there because K % 256 != 0."""
    need_gpu()
    rng = np.random.default_rng(M + N + K)
    a = (*_rand_packed(rng, M, K, 0x00, 0x7E), np.float32(0.7))
    b = (*_rand_packed(rng, N, K, 0x00, 0x7E), np.float32(1.3))
    note(f"mid-M tile config M={M} N={N} K={K}")
    y = np_(_gemm(to_gpu(*a), to_gpu(*b), "bf16"))
    y_ref, bound = gemm_ref(*a, *b)
    ok, worst = check_gemm(y, y_ref, bound, "bf16")
    assert ok, worst


@pytest.mark.parametrize("M,N", [(65, 96), (100, 40), (128, 200)])
def test_decode_two_passes(M, N):
    """65 <= M <= 128 runs the weight-streaming kernel in two 64-row passes
    when 64 x 64 MFMA tiles would not fill the chip (small N here)."""
    need_gpu()
    K = 512
    rng = np.random.default_rng(M + N)
    a = (*_rand_packed(rng, M, K, 0x00, 0x7E), np.float32(0.7))
    b = (*_rand_packed(rng, N, K, 0x00, 0x7E), np.float32(1.3))
    for out in ("f32", "bf16"):
        note(f"decode two passes M={M} N={N} out={out}")
        y = np_(_gemm(to_gpu(*a), to_gpu(*b), out))
        y_ref, bound = gemm_ref(*a, *b)
        ok, worst = check_gemm(y, y_ref, bound, out)
        assert ok, (out, worst)


@pytest.mark.parametrize("M", list(range(1, 65)))
def test_every_small_m(M):
    need_gpu()
    rng = np.random.default_rng(M)
    K, N = 512, 200
    a = (*_rand_packed(rng, M, K), np.float32(0.03))
    b = (*_rand_packed(rng, N, K), np.float32(0.5))
    y = np_(_gemm(to_gpu(*a), to_gpu(*b), "f32"))
    y_ref, bound = gemm_ref(*a, *b)
    ok, worst = check_gemm(y, y_ref, bound, "f32")
    assert ok, worst


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 128), (7, 129, 384), (300, 260, 256), (257, 255, 1024), (33, 96, 48),
    (5, 7, 16), (129, 3, 2048), (600, 520, 640), (64, 64, 8192),
    (3, 1000, 2560), (32, 33, 256), (17, 4100, 1024), (31, 70, 16384), (2, 31, 768),
])
def test_odd_shapes(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M * 7 + N + K)
    a = (*_rand_packed(rng, M, K, 0x00, 0x7E), np.float32(0.7))
    b = (*_rand_packed(rng, N, K, 0x00, 0x7E), np.float32(1.3))
    for out in ("f32", "bf16"):
        note(f"odd shape M={M} N={N} K={K} out={out}")
        y = np_(_gemm(to_gpu(*a), to_gpu(*b), out))
        y_ref, bound = gemm_ref(*a, *b)
        ok, worst = check_gemm(y, y_ref, bound, out)
        assert ok, (out, worst)


def test_k_zero_gives_zeros():
    need_gpu()
    dev = "cuda"
    e = torch.empty((4, 0), dtype=torch.uint8, device=dev)
    g = torch.ones(1, device=dev)
    y = torch.full((4, 6), 7.0, device=dev)
    st = nv.nvfp4_gemm_raw(4, 6, 0, e.data_ptr(), e.data_ptr(), g.data_ptr(), e.data_ptr(),
                           e.data_ptr(), g.data_ptr(), y.data_ptr(), nv.NVFP4_F32, 6)
    assert st == nv.NVFP4_OK
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0


def test_bf16_output_is_rne_of_f32_and_repeatable():
    need_gpu()
    rng = np.random.default_rng(1)
    for M in (4, 32, 300):
        a = to_gpu(*_rand_packed(rng, M, 1024), np.float32(0.01))
        b = to_gpu(*_rand_packed(rng, 384, 1024), np.float32(0.2))
        y32 = _gemm(a, b, "f32")
        y16 = _gemm(a, b, "bf16")
        assert torch.equal(y32.to(torch.bfloat16), y16)
        assert torch.equal(_gemm(a, b, "f32"), y32)


def test_linear_workload_full():
    """M=4096, N=K=8192 bf16 inputs quantised on the GPU, every byte and both
    global scales checked against the oracle; the whole bf16 output of the
    GEMM (the launch configuration the bench times) against the fp64 oracle
    GEMM."""
    need_gpu()
    x_cpu, w_cpu = wl.gemm_inputs(1, wl.LINEAR)
    note("linear workload quantize")
    a = nv.nvfp4_quantize(x_cpu.cuda())
    b = nv.nvfp4_quantize(w_cpu.cuda())
    note("linear workload gemm")
    y = _gemm(a, b, "bf16")
    note("linear workload: oracle quantise of x and W")
    ra = oracle_quantize(x_cpu)
    rb = oracle_quantize(w_cpu)
    assert_bytes_equal(*a, *ra)
    assert_bytes_equal(*b, *rb)
    note("linear workload: oracle GEMM (fp64, full output)")
    y_ref, bound = gemm_ref(*ra, *rb)
    ok, worst = check_gemm(np_(y), y_ref, bound, "bf16")
    assert ok, worst


def _rows_of(packed, rows):
    q, s, g = packed
    idx = torch.from_numpy(np.asarray(rows)).to(q.device)
    return np_(q.index_select(0, idx)), np_(s.index_select(0, idx))


def test_large_outlier_workload():
    """M = N = K = 16384 with 1 % x50 outliers, quantised on the GPU.  The
    oracle quantises all of x and W (row chunks; global scales from the whole
    tensors) and every byte must match.  The bf16 GEMM output is checked in
    full over K on 64 random rows, 64 random columns and 4096 random
    elements."""
    need_gpu()
    c = wl.LARGE
    x_cpu, w_cpu = wl.gemm_inputs(4, c)
    note("large workload quantize")
    a = nv.nvfp4_quantize(x_cpu.cuda())
    b = nv.nvfp4_quantize(w_cpu.cuda())
    note("large workload gemm")
    y = _gemm(a, b, "bf16")
    ref = {}
    for name, t_cpu, got in (("x", x_cpu, a), ("W", w_cpu, b)):
        g = oracle_global_scale(t_cpu)
        assert np.float32(np_(got[2])[0]) == g, name
        qs, ss = [], []
        for r0 in range(0, t_cpu.shape[0], 2048):
            note(f"large workload: oracle quantise of {name} rows {r0}..{r0 + 2047}")
            rq, rs, _ = oracle_quantize(t_cpu[r0:r0 + 2048], g)
            gq, gs = _rows_of(got, range(r0, min(r0 + 2048, t_cpu.shape[0])))
            assert np.array_equal(gq, rq) and np.array_equal(gs, rs), (name, r0)
            qs.append(rq)
            ss.append(rs)
        ref[name] = (np.concatenate(qs), np.concatenate(ss), g)
    rq_x, rs_x, gx = ref["x"]
    rq_w, rs_w, gw = ref["W"]
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(c.M, 64, replace=False))
    cols = np.sort(rng.choice(c.N, 64, replace=False))
    y_np = np_(y)
    note("large workload: oracle GEMM on 64 full rows")
    y_ref, bound = gemm_ref(rq_x[rows], rs_x[rows], gx, rq_w, rs_w, gw)
    ok, worst = check_gemm(y_np[rows], y_ref, bound, "bf16")
    assert ok, ("rows", worst)
    note("large workload: oracle GEMM on 64 full columns")
    y_ref, bound = gemm_ref(rq_x, rs_x, gx, rq_w[cols], rs_w[cols], gw)
    ok, worst = check_gemm(y_np[:, cols], y_ref, bound, "bf16")
    assert ok, ("cols", worst)
    note("large workload: oracle GEMM on 4096 random elements")
    em = rng.integers(0, c.M, 4096)
    en = rng.integers(0, c.N, 4096)
    for i0 in range(0, 4096, 512):
        m, n = em[i0:i0 + 512], en[i0:i0 + 512]
        xa = dequantize_ref(rq_x[m], rs_x[m])
        wb = dequantize_ref(rq_w[n], rs_w[n])
        alpha = float(np.float64(gx) * np.float64(gw))
        y_ref = np.einsum("ik,ik->i", xa, wb) * alpha
        bound = np.einsum("ik,ik->i", np.abs(xa), np.abs(wb)) * abs(alpha)
        ok, worst = check_gemm(y_np[m, n], y_ref, bound, "bf16")
        assert ok, ("elements", i0, worst)


@pytest.mark.parametrize("out,pad,shift", [("bf16", 8, 0), ("bf16", 3, 0), ("bf16", 8, 1),
                                           ("f32", 5, 0), ("f32", 4, 1)])
def test_strided_output_writers(out, pad, shift):
    """y written into a wider buffer (row stride N + pad, start shifted by
    `shift` elements): whole 256 x 256 tiles take the staged 16-byte writer
    (bf16, 16-byte aligned rows) or the per-element one (odd stride, shifted
    start, fp32), edge tiles the checked one; the padding keeps its
    sentinel."""
    need_gpu()
    M, N, K = 4096 + 40, 4096 + 24, 128
    rng = np.random.default_rng(pad * 10 + shift)
    a = (*_rand_packed(rng, M, K, 0x20, 0x48), np.float32(0.5))
    b = (*_rand_packed(rng, N, K, 0x20, 0x48), np.float32(0.25))
    code_dt = torch.bfloat16 if out == "bf16" else torch.float32
    ld = N + pad
    buf = torch.full((M * ld + shift + pad,), -7.0, dtype=code_dt, device="cuda")
    y = buf[shift:shift + M * ld].view(M, ld)[:, :N]
    note(f"strided output out={out} ld_y={ld} shift={shift}")
    nv.nvfp4_gemm(to_gpu(*a), to_gpu(*b), out_dtype=out, y=y)
    torch.cuda.synchronize()
    y_ref, bound = gemm_ref(*a, *b)
    ok, worst = check_gemm(np_(y.contiguous()), y_ref, bound, out)
    assert ok, worst
    full = buf.float().cpu().numpy()
    mask = np.ones(full.shape, bool)
    idx = shift + (np.arange(M)[:, None] * ld + np.arange(N)[None, :])
    mask[idx.ravel()] = False
    assert np.all(full[mask] == -7.0), "writes outside the output view"


@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (300, 384, 1024), (4096, 256, 128), (37, 48, 48)])
@pytest.mark.parametrize("ga,gb", [(1e-30, 1e-12), (1e-30, 1e-15), (3e18, 3e18)])
def test_bf16_output_rne_at_the_extremes(M, N, K, ga, gb):
    """Global scales whose product is subnormal (outputs near or below the
    smallest normal fp32) or huge (outputs overflow to infinity): the bf16
    output still equals round-to-nearest-even of the fp32 output, on the
    decode, MFMA (whole and edge tiles) and general kernels."""
    need_gpu()
    rng = np.random.default_rng(M + N)
    a = to_gpu(*_rand_packed(rng, M, K, 0x30, 0x48), np.float32(ga))
    b = to_gpu(*_rand_packed(rng, N, K, 0x30, 0x48), np.float32(gb))
    note(f"bf16 extremes M={M} N={N} K={K} ga={ga} gb={gb}")
    y32 = _gemm(a, b, "f32")
    y16 = _gemm(a, b, "bf16")
    ref = y32.cpu().to(torch.bfloat16)
    assert torch.equal(ref.view(torch.int16), y16.cpu().view(torch.int16))


def test_operands_beyond_4_gib():
    """Maximum sizes: a 600000 x 16384 operand packs to 4.9 GB, so its byte
    offsets pass 2^31 and 2^32.  The quantiser walks it with 64-bit offsets,
    and the GEMM sends it to the general kernel both as A (against 40 weight
    rows, f32 out) and as W (under 3 activation rows, bf16 out).  Rows repeat
    a seeded 1000-row block; 1000 divides neither 2^31 nor 2^32 bytes' worth
    of rows (8192 bytes each), so an offset that wrapped would read another
    block row.  Rows on both sides of those offsets, the last rows and a
    random sample are checked: quantised bytes exactly, GEMM outputs to the
    tolerance."""
    need_gpu()
    rows, K, period = 600000, 16384, 1000
    block = wl.randn((period, K), 8101, "bf16")
    g = oracle_global_scale(block)                   # the tensor's amax is the block's
    note(f"quantise {rows} x {K} bf16 ({rows * K * 2 / 1e9:.1f} GB)")
    x = block.cuda().repeat(rows // period, 1)
    big = nv.nvfp4_quantize(x)
    torch.cuda.synchronize()
    del x
    torch.cuda.empty_cache()
    per_row = K // 2
    edges = [0, 1, (1 << 31) // per_row - 1, (1 << 31) // per_row,
             (1 << 32) // per_row - 1, (1 << 32) // per_row, rows - 2, rows - 1]
    rng = np.random.default_rng(8102)
    sample = np.unique(np.concatenate([edges, rng.choice(rows, 8, replace=False)]))
    idx = torch.from_numpy(sample).cuda()
    ra = oracle_quantize(block[torch.from_numpy(sample % period)], g)
    assert_bytes_equal(big[0][idx], big[1][idx], big[2], *ra)

    rb = oracle_quantize(wl.randn((40, K), 8103, "bf16"))
    note(f"gemm A beyond 4 GiB M={rows} N=40 K={K} (general kernel)")
    y = _gemm(big, to_gpu(*rb), "f32")
    y_ref, bound = gemm_ref(*ra, *rb)
    ok, worst = check_gemm(np_(y[idx]), y_ref, bound, "f32")
    assert ok, f"A beyond 4 GiB: worst |err|/tol = {worst}"
    del y

    rx = oracle_quantize(wl.randn((3, K), 8104, "bf16"))
    note(f"gemm W beyond 4 GiB M=3 N={rows} K={K} (general kernel)")
    y = _gemm(to_gpu(*rx), big, "bf16")
    y_ref, bound = gemm_ref(*rx, *ra)
    ok, worst = check_gemm(np_(y[:, idx]), y_ref, bound, "bf16")
    assert ok, f"W beyond 4 GiB: worst |err|/tol = {worst}"


def test_general_kernel_past_its_row_chunks():
    """Dense calls with K = 48 run the general kernel, which launches at most
    1,048,560 rows at a time: 1,100,000 rows (a seeded 1000-row block
    repeated) cross that boundary.  The fp32 output is checked on rows
    around it, the last rows and a random sample; the NVFP4 output of the
    same call equals the oracle's quantisation of that fp32 output under the
    same static scale on those rows."""
    need_gpu()
    M, K, N, period = 1_100_000, 48, 32, 1000
    ra = oracle_quantize(wl.randn((period, K), 8301, "bf16"))
    rb = oracle_quantize(wl.randn((N, K), 8302, "bf16"))
    a_small = to_gpu(*ra)
    a = (a_small[0].repeat(M // period, 1), a_small[1].repeat(M // period, 1), a_small[2])
    rng = np.random.default_rng(8303)
    rows = np.unique(np.concatenate([[0, 1_048_559, 1_048_560, 1_048_561, M - 2, M - 1],
                                     rng.choice(M, 8, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    note(f"dense general kernel M={M} N={N} K={K}")
    y = _gemm(a, to_gpu(*rb), "f32")
    y_rows = np_(y[idx])
    y_ref, bound = gemm_ref(ra[0][rows % period], ra[1][rows % period], ra[2], *rb)
    ok, worst = check_gemm(y_rows, y_ref, bound, "f32")
    assert ok, worst
    g = torch.tensor([float(np.abs(y_rows).max() / 2688.0)], dtype=torch.float32, device="cuda")
    note(f"dense general kernel, NVFP4 output, M={M}")
    q, s, _ = nv.nvfp4_gemm_nvfp4_out(a, to_gpu(*rb), g)
    torch.cuda.synchronize()
    ref = oracle_quantize(torch.from_numpy(y_rows), np.float32(g.item()))
    assert_bytes_equal(q[idx], s[idx], g, *ref)


def test_binding_checks_outputs_and_packs_operands():
    """The quantiser returns checked Packed operands; an output buffer of the
    wrong dtype, shape or layout is refused before the library is called."""
    need_gpu()
    x = wl.randn((8, 64), 8401, "bf16").cuda()
    w = wl.randn((32, 64), 8402, "bf16").cuda()
    a, b = nv.nvfp4_quantize(x), nv.nvfp4_quantize(w)
    assert type(a) is nv.Packed and (a.rows, a.K) == (8, 64)
    for y, dt in ((torch.empty((8, 32), dtype=torch.bfloat16, device="cuda"), "f32"),
                  (torch.empty((8, 33), dtype=torch.float32, device="cuda"), "f32"),
                  (torch.empty((32, 8), dtype=torch.float32, device="cuda").t(), "f32"),
                  (torch.empty((8, 32), dtype=torch.float32), "f32")):
        with pytest.raises(ValueError):
            nv.nvfp4_gemm(a, b, dt, y=y)
    with pytest.raises(ValueError):   # operands of different K
        nv.nvfp4_gemm(a, nv.nvfp4_quantize(wl.randn((32, 128), 8403, "bf16").cuda()), "f32")
    y = nv.nvfp4_gemm(tuple(a), tuple(b), "f32")     # plain tuples are checked and accepted
    torch.cuda.synchronize()
    assert y.shape == (8, 32)
