"""GPU parity of the decode path (up to 32 tokens, K a multiple of 1024: the
LDS-ring weight-streaming kernel) against the oracle, through the C ABI.

Operands are packed directly (random nibbles and scale bytes) or quantised by
the oracle, so the GEMM is checked independently of the GPU quantiser.
Tolerance: |y - y_ref| <= 1e-5 * sum_k |x_k w_k| per element, plus one bf16
ulp for bf16 output.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from oracle import check_gemm, dequantize_ref, gemm_ref, pack_nibbles, quantize_ref
from tests.gpu_util import need_gpu, note, np_, to_gpu

pytestmark = pytest.mark.gpu


def _rand_packed(rng, rows, K, lo=0x00, hi=0x7E):
    q = rng.integers(0, 256, size=(rows, K // 2)).astype(np.uint8)
    s = rng.integers(lo, hi + 1, size=(rows, K // 16)).astype(np.uint8)
    return q, s


def _run(a, b, out):
    y = nv.nvfp4_gemm(to_gpu(*a), to_gpu(*b), out_dtype=out)
    torch.cuda.synchronize()
    return np_(y)


@pytest.mark.parametrize("K,N", [(1024, 200), (3072, 97), (2048, 32)])
def test_every_m_up_to_32(K, N):
    """Every token count 1..32 (each ring depth and token-fragment count),
    ragged and exact weight-row tiles, fp32 and bf16 output."""
    need_gpu()
    rng = np.random.default_rng(K + N)
    b = (*_rand_packed(rng, N, K), np.float32(0.75))
    for M in range(1, 33):
        a = (*_rand_packed(rng, M, K), np.float32(0.03))
        y_ref, bound = gemm_ref(*a, *b)
        for out in ("f32", "bf16"):
            note(f"decode M={M} N={N} K={K} out={out}")
            ok, worst = check_gemm(_run(a, b, out), y_ref, bound, out)
            assert ok, (M, out, worst)


@pytest.mark.parametrize("N", [1, 5, 31, 33, 100])
def test_few_weight_rows(N):
    """Fewer weight rows than one workgroup's 32, or a ragged last tile."""
    need_gpu()
    rng = np.random.default_rng(N)
    K = 1024
    b = (*_rand_packed(rng, N, K), np.float32(1.5))
    for M in (1, 7, 16, 32):
        a = (*_rand_packed(rng, M, K), np.float32(0.5))
        note(f"decode few rows M={M} N={N}")
        y_ref, bound = gemm_ref(*a, *b)
        ok, worst = check_gemm(_run(a, b, "f32"), y_ref, bound, "f32")
        assert ok, (M, worst)


@pytest.mark.parametrize("M", [1, 5, 16, 32])
def test_exhaustive_dequant_identity(M):
    """W [16, 1024]: each 16-element block holds all 16 nibbles, and the 1024
    blocks carry every finite scale byte (4 times).  A holds M one-hot rows
    (nibble 1.0, scale 1.0, g = 1); over 1024 / M launches the one-hot
    positions cover all of K, so y reads back every W element, i.e. every
    nibble under every scale byte through the kernel, bit for bit."""
    need_gpu()
    N, K = 16, 1024
    rng = np.random.default_rng(M)
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x3F, 0xBF                 # NaN codes replaced
    perm = np.argsort(rng.random((N * K // 16, 16)), axis=1).astype(np.uint8)
    b = (pack_nibbles(perm.reshape(N, K)), np.resize(codes, N * K // 16).reshape(N, K // 16),
         np.float32(1))
    w_dq = dequantize_ref(b[0], b[1]).astype(np.float32)   # every value exact in fp32
    order = rng.permutation(K)
    note(f"decode exhaustive dequant M={M}")
    for start in range(0, K, M):
        ks = order[start:start + M]
        m = len(ks)
        nib = np.zeros((m, K), dtype=np.uint8)
        nib[np.arange(m), ks] = 0x2
        a = (pack_nibbles(nib), np.full((m, K // 16), 0x38, np.uint8), np.float32(1))
        y = _run(a, b, "f32")
        assert np.array_equal(y, w_dq[:, ks].T), f"positions {ks[:4]}..."


@pytest.mark.parametrize("out,pad", [("bf16", 8), ("bf16", 3), ("f32", 5)])
def test_strided_output(out, pad):
    """y written into a wider buffer: the padding keeps its sentinel."""
    need_gpu()
    M, N, K = 20, 300, 2048
    rng = np.random.default_rng(pad)
    a = (*_rand_packed(rng, M, K, 0x20, 0x48), np.float32(0.5))
    b = (*_rand_packed(rng, N, K, 0x20, 0x48), np.float32(0.25))
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    ld = N + pad
    buf = torch.full((M, ld), -7.0, dtype=dt, device="cuda")
    note(f"decode strided output out={out} ld_y={ld}")
    nv.nvfp4_gemm(to_gpu(*a), to_gpu(*b), out_dtype=out, y=buf[:, :N])
    torch.cuda.synchronize()
    y_ref, bound = gemm_ref(*a, *b)
    full = np_(buf)
    ok, worst = check_gemm(full[:, :N], y_ref, bound, out)
    assert ok, worst
    assert np.all(full[:, N:] == -7.0), "writes outside the output view"


@pytest.mark.parametrize("ga,gb", [(1e-30, 1e-12), (3e18, 3e18)])
def test_bf16_rne_at_the_extremes(ga, gb):
    """Subnormal and overflowing global-scale products: bf16 output equals
    round-to-nearest-even of the fp32 output bit for bit."""
    need_gpu()
    rng = np.random.default_rng(3)
    a = to_gpu(*_rand_packed(rng, 16, 1024, 0x30, 0x48), np.float32(ga))
    b = to_gpu(*_rand_packed(rng, 512, 1024, 0x30, 0x48), np.float32(gb))
    y32 = nv.nvfp4_gemm(a, b, "f32")
    y16 = nv.nvfp4_gemm(a, b, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(y32.cpu().to(torch.bfloat16).view(torch.int16), y16.cpu().view(torch.int16))


def test_repeatable_bitwise():
    need_gpu()
    rng = np.random.default_rng(9)
    a = to_gpu(*_rand_packed(rng, 32, 4096), np.float32(0.1))
    b = to_gpu(*_rand_packed(rng, 1000, 4096), np.float32(0.2))
    y0 = nv.nvfp4_gemm(a, b, "f32")
    y1 = nv.nvfp4_gemm(a, b, "f32")
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("M", [1, 16, 32])
def test_decode_workload_full_output(M):
    """The decode workload (N = K = 8192, bf16 inputs quantised on the GPU,
    bytes checked against the oracle) in the launch configuration the bench
    times: the whole bf16 output against the fp64 oracle GEMM."""
    need_gpu()
    cfg = wl.DECODE[M]
    x_cpu, w_cpu = wl.gemm_inputs(2, cfg)
    note(f"decode workload M={M}: quantise")
    a = nv.nvfp4_quantize(x_cpu.cuda())
    b = nv.nvfp4_quantize(w_cpu.cuda())
    note(f"decode workload M={M}: gemm")
    y = nv.nvfp4_gemm(a, b, "bf16")
    torch.cuda.synchronize()
    ra = quantize_ref(np_(x_cpu))
    rb = quantize_ref(np_(w_cpu))
    for got, ref in ((a, ra), (b, rb)):
        assert np.array_equal(np_(got[0]), ref[0]) and np.array_equal(np_(got[1]), ref[1])
        assert np.float32(np_(got[2])[0]) == ref[2]
    y_ref, bound = gemm_ref(*ra, *rb)
    ok, worst = check_gemm(np_(y), y_ref, bound, "bf16")
    assert ok, worst


# ---------------------------------------------------------------------------
# whole-row weight stream (up to 4 tokens at K = 8192; the other shapes here
# run the LDS-tile kernel, checked the same way)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K", [4096, 8192])
@pytest.mark.parametrize("N", [2102, 20, 3])
def test_rows_every_m_up_to_16(K, N):
    """Every token count 1..16 (the whole-row kernel for up to 4 tokens at
    K = 8192, the LDS-tile kernel otherwise), N ragged against 4-row chunks
    and spanning several chunks per workgroup (2102) or fewer row groups
    than workgroups (20, 3), fp32 and bf16 output; y of the first M rows of
    one 16-row activation against one oracle GEMM."""
    need_gpu()
    rng = np.random.default_rng(K + N)
    b = (*_rand_packed(rng, N, K), np.float32(0.75))
    a = (*_rand_packed(rng, 16, K), np.float32(0.03))
    y_ref, bound = gemm_ref(*a, *b)
    ga, gb = to_gpu(*a), to_gpu(*b)
    for M in range(1, 17):
        am = (ga[0][:M], ga[1][:M], ga[2])
        for out in ("f32", "bf16"):
            note(f"decode rows M={M} N={N} K={K} out={out}")
            y = nv.nvfp4_gemm(am, gb, out_dtype=out)
            torch.cuda.synchronize()
            ok, worst = check_gemm(np_(y), y_ref[:M], bound[:M], out)
            assert ok, (M, out, worst)


@pytest.mark.parametrize("M,K", [(4, 8192), (1, 8192), (16, 8192), (8, 4096)])
def test_rows_exhaustive_dequant_identity(M, K):
    """W [16, K]: each 16-element block holds all 16 nibbles and the blocks
    carry every finite scale byte in turn.  Launch i multiplies M one-hot
    activation rows (nibble 1.0 at K-positions perm[M i .. M i + M - 1],
    scale 1.0, g = 1), so over K / M launches every W element, i.e. every
    nibble under every scale byte at every K position, is read back through
    the kernel bit for bit."""
    need_gpu()
    N = 16
    rng = np.random.default_rng(M * K)
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x3F, 0xBF                 # NaN codes replaced
    perm16 = np.argsort(rng.random((N * K // 16, 16)), axis=1).astype(np.uint8)
    b = (pack_nibbles(perm16.reshape(N, K)), np.resize(codes, N * K // 16).reshape(N, K // 16),
         np.float32(1))
    w_dq = dequantize_ref(b[0], b[1]).astype(np.float32)
    order = rng.permutation(K)
    nib = np.zeros((K, K), dtype=np.uint8)
    nib[np.arange(K), order] = 0x2                          # row j: one-hot at order[j]
    a_q = torch.from_numpy(pack_nibbles(nib)).cuda()
    a_s = torch.full((K, K // 16), 0x38, dtype=torch.uint8, device="cuda")
    a_g = torch.ones(1, dtype=torch.float32, device="cuda")
    gb = to_gpu(*b)
    launches = K // M
    y_all = torch.empty((launches, M, N), dtype=torch.float32, device="cuda")
    note(f"decode rows exhaustive dequant M={M} K={K}: {launches} launches")
    for i in range(launches):
        nv.nvfp4_gemm((a_q[M * i:M * i + M], a_s[M * i:M * i + M], a_g), gb, "f32", y=y_all[i])
    torch.cuda.synchronize()
    got = np_(y_all).reshape(K, N)                          # row j = W_dq[:, order[j]]
    assert np.array_equal(got, w_dq[:, order].T)


def test_rows_strided_and_repeatable():
    """Output rows with a stride (padding untouched), bitwise repeat, and
    bf16 = round-to-nearest-even of fp32 on the whole-row kernel."""
    need_gpu()
    M, N, K = 12, 700, 8192
    rng = np.random.default_rng(5)
    a = (*_rand_packed(rng, M, K, 0x20, 0x48), np.float32(0.5))
    b = (*_rand_packed(rng, N, K, 0x20, 0x48), np.float32(0.25))
    ga, gb = to_gpu(*a), to_gpu(*b)
    buf = torch.full((M, N + 5), -7.0, dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm(ga, gb, "f32", y=buf[:, :N])
    y2 = nv.nvfp4_gemm(ga, gb, "f32")
    y16 = nv.nvfp4_gemm(ga, gb, "bf16")
    torch.cuda.synchronize()
    full = np_(buf)
    assert np.all(full[:, N:] == -7.0)
    assert torch.equal(buf[:, :N], y2)
    assert torch.equal(y2.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))
    y_ref, bound = gemm_ref(*a, *b)
    ok, worst = check_gemm(full[:, :N], y_ref, bound, "f32")
    assert ok, worst


@pytest.mark.parametrize("M,N", [(4, 44032), (4, 44036), (1, 44036)])
def test_rows_very_wide_output(M, N):
    """K = 8192: the whole-row kernel parks every chunk's partial sums in LDS
    until the end, which holds 43 chunks of 4 rows (N = 44032 on 256
    compute units); one more row group sends the call to the tile kernel.
    Both sides of the boundary are checked on sampled output columns, the
    last ones included."""
    need_gpu()
    K = 8192
    rng = np.random.default_rng(N)
    a = (*_rand_packed(rng, M, K, 0x20, 0x48), np.float32(0.5))
    bq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bs = rng.integers(0x20, 0x49, size=(N, K // 16), dtype=np.uint8)
    note(f"decode rows very wide M={M} N={N}")
    y = nv.nvfp4_gemm(to_gpu(*a), to_gpu(bq, bs, np.float32(0.25)), "f32")
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([rng.choice(N, 120, replace=False), np.arange(N - 8, N)]))
    y_ref, bound = gemm_ref(*a, bq[cols], bs[cols], np.float32(0.25))
    ok, worst = check_gemm(np_(y)[:, cols], y_ref, bound, "f32")
    assert ok, worst
