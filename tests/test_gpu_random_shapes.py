"""Seeded random shapes across the whole dispatch space, every entry point
against the oracle: dense GEMM (fp32 and bf16 output), the NVFP4-output GEMM
(bytes equal to the oracle's quantisation of the fp32 result) and the grouped
GEMM (with and without a routing index).  M, N and K are drawn so that each
kernel (decode in one or two passes, the three MFMA tile configurations,
the streaming grouped kernel and the general kernels) gets ragged shapes;
sizes stay small enough for the fp64 oracle."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from oracle import check_gemm, gemm_ref, grouped_gemm_ref, quantize_ref
from tests.gpu_util import need_gpu, note, np_, to_gpu

pytestmark = pytest.mark.gpu


def _packed(rng, rows, K):
    q = rng.integers(0, 256, size=(rows, K // 2)).astype(np.uint8)
    s = rng.integers(0x18, 0x50, size=(rows, K // 16)).astype(np.uint8)
    return q, s


def _dense_shape(rng, i):
    kind = i % 4
    if kind == 0:     # decode kernel
        M = int(rng.integers(1, 129))
        K = 256 * int(rng.integers(1, 9))
        N = 16 * int(rng.integers(1, 80))
    elif kind == 1:   # MFMA tiles
        M = int(rng.integers(129, 700))
        K = 128 * int(rng.integers(1, 7))
        N = 16 * int(rng.integers(8, 120))
    elif kind == 2:   # general kernel (K not a multiple of 128 and, for M <= 128, of 256)
        M = int(rng.integers(1, 300))
        K = 16 * int(rng.choice([1, 3, 5, 7, 9, 11, 13, 15, 17, 23]))
        N = 16 * int(rng.integers(1, 40))
    else:             # decode K but M above the decode range -> MFMA or general
        M = int(rng.integers(100, 400))
        K = 16 * int(rng.integers(1, 40))
        N = 16 * int(rng.integers(1, 60))
    return M, N, K


@pytest.mark.parametrize("i", range(24))
def test_dense_random(i):
    need_gpu()
    rng = np.random.default_rng(1000 + i)
    M, N, K = _dense_shape(rng, i)
    a = (*_packed(rng, M, K), np.float32(rng.uniform(0.01, 2.0)))
    b = (*_packed(rng, N, K), np.float32(rng.uniform(0.01, 2.0)))
    ga, gb = to_gpu(*a), to_gpu(*b)
    note(f"random dense #{i} M={M} N={N} K={K}")
    y_ref, bound = gemm_ref(*a, *b)
    y32 = nv.nvfp4_gemm(ga, gb, out_dtype="f32")
    y16 = nv.nvfp4_gemm(ga, gb, out_dtype="bf16")
    torch.cuda.synchronize()
    ok, worst = check_gemm(np_(y32), y_ref, bound, "f32")
    assert ok, worst
    assert torch.equal(y32.to(torch.bfloat16), y16)
    y_np = np_(y32)
    g = np.float32(np.abs(y_np).max() / np.float32(2688.0) * np.float32(rng.uniform(0.5, 1.5)))
    q, s, _ = nv.nvfp4_gemm_nvfp4_out(ga, gb, torch.tensor([float(g)], device="cuda"))
    torch.cuda.synchronize()
    rq, rs, _ = quantize_ref(y_np, global_scale=g)
    assert np.array_equal(np_(s), rs) and np.array_equal(np_(q), rq)


@pytest.mark.parametrize("i", range(12))
def test_grouped_random(i):
    need_gpu()
    rng = np.random.default_rng(2000 + i)
    G = int(rng.integers(1, 12))
    counts = [int(c) if rng.random() > 0.2 else 0 for c in rng.integers(1, 70, size=G)]
    counts[-1] = max(counts[-1], 1)
    K = 512 * int(rng.integers(1, 4)) if i % 3 else 16 * int(rng.integers(1, 40))
    N = 16 * int(rng.integers(1, 24)) + (0 if i % 2 else 8)
    off = wl.ragged_offsets(counts)
    total = int(off[-1])
    a_rows = int(rng.integers(1, 60))
    aq, as_ = _packed(rng, a_rows, K)
    ag = np.float32(0.3)
    bq, bs = _packed(rng, G * N, K)
    bq, bs = bq.reshape(G, N, K // 2), bs.reshape(G, N, K // 16)
    bg = rng.uniform(0.2, 1.5, size=G).astype(np.float32)
    idx = rng.integers(-2, a_rows + 2, size=total).astype(np.int32)
    valid = (idx >= 0) & (idx < a_rows)
    gq = np.where(valid[:, None], aq[np.clip(idx, 0, a_rows - 1)], 0).astype(np.uint8)
    gs = np.where(valid[:, None], as_[np.clip(idx, 0, a_rows - 1)], 0).astype(np.uint8)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    note(f"random grouped #{i} G={G} counts={counts} N={N} K={K} a_rows={a_rows}")
    y_ref, bound = grouped_gemm_ref(off.numpy(), gq, gs, ag, bq, bs, bg)
    for out in ("f32", "bf16"):
        # through the index, and on the rows gathered beforehand
        y = nv.nvfp4_grouped_gemm(off.to(dev), total, (t(aq), t(as_), torch.tensor([ag], device=dev)),
                                  (t(bq), t(bs), t(bg)), out_dtype=out, row_index=t(idx))
        y2 = nv.nvfp4_grouped_gemm(off.to(dev), total, (t(gq), t(gs), torch.tensor([ag], device=dev)),
                                   (t(bq), t(bs), t(bg)), out_dtype=out)
        torch.cuda.synchronize()
        for yy in (y, y2):
            ok, worst = check_gemm(np_(yy), y_ref, bound, out)
            assert ok, (out, worst)
