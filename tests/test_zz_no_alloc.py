"""nvfp4_quantize_noalloc (the quantiser for callers that cannot allocate:
its amax workspace is the library's own per-GPU device array) against
nvfp4_quantize with a caller-given workspace, through the C ABI: identical
bytes and global scale on two calls in a row, the second with a smaller
input, then with a static scale."""
import ctypes

import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from tests.gpu_util import need_gpu, note

pytestmark = pytest.mark.gpu


def _reference(x, global_scale=None):
    return nv.nvfp4_quantize(x, global_scale=global_scale)


def _noalloc(x, global_scale=None):
    rows, cols = x.shape
    q = torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device=x.device)
    s = torch.full((rows, cols // 16), 0xCD, dtype=torch.uint8, device=x.device)
    g = torch.full((1,), -1.0, dtype=torch.float32, device=x.device)
    flags = 0
    if global_scale is not None:
        g.copy_(global_scale)
        flags = nv.NVFP4_GLOBAL_SCALE_GIVEN
    dt = nv.NVFP4_BF16 if x.dtype == torch.bfloat16 else nv.NVFP4_F32
    torch.cuda.synchronize()                      # buffers ready before the raw call
    st = nv.nvfp4_quantize_noalloc_raw(x.data_ptr(), dt, rows, cols, x.stride(0), q.data_ptr(),
                                       s.data_ptr(), g.data_ptr(), flags)
    assert st == nv.NVFP4_OK, st
    return q, s, g


def _same(a, b):
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_noalloc_matches_workspace_entry_point():
    need_gpu()
    big = wl.randn((4096, 8192), 9101, "bf16", True).cuda()      # 1024 amax partials
    small = wl.randn((37, 256), 9102, "fp32").cuda()             # 1 partial
    note("no-alloc quantise: 4096 x 8192 bf16")
    got_big = _noalloc(big)
    torch.cuda.synchronize()
    _same(got_big, _reference(big))
    note("no-alloc quantise: 37 x 256 fp32 (second call, smaller)")
    got_small = _noalloc(small)
    torch.cuda.synchronize()
    _same(got_small, _reference(small))
    gs = torch.tensor([0.004], dtype=torch.float32, device="cuda")
    note("no-alloc quantise: static scale")
    got_static = _noalloc(small, gs)
    torch.cuda.synchronize()
    _same(got_static, _reference(small, gs))


def test_noalloc_rejects_bad_arguments_before_launch():
    need_gpu()
    x = torch.zeros((4, 32), dtype=torch.float32, device="cuda")
    q = torch.empty((4, 16), dtype=torch.uint8, device="cuda")
    s = torch.empty((4, 2), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    st = nv.nvfp4_quantize_noalloc_raw(x.data_ptr(), nv.NVFP4_F32, 4, 24, 32, q.data_ptr(),
                                       s.data_ptr(), g.data_ptr(), 0)
    assert st == nv.NVFP4_ERR_INVALID_ARG
    st = nv.nvfp4_quantize_noalloc_raw(x.data_ptr(), nv.NVFP4_F32, 4, 32, 32, q.data_ptr(),
                                       s.data_ptr(), None, 0)
    assert st == nv.NVFP4_ERR_INVALID_ARG
