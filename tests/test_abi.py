"""C-ABI checks that need no GPU: the library loads, exports every function
include/nvfp4.h declares, and rejects invalid arguments on the host before
anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

# Fake, never-dereferenced device addresses (validation fails before use).
P16 = ctypes.c_void_p(0x10000)
P8 = ctypes.c_void_p(0x10008)
P4 = ctypes.c_void_p(0x10004)
NULL = None


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = nv.load()
    declared = _declared_functions()
    assert set(declared) == set(nv.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = nv.load()
    assert lib.nvfp4_status_string(0) == b"NVFP4_OK"
    assert lib.nvfp4_status_string(-1) == b"NVFP4_ERR_INVALID_ARG"
    assert lib.nvfp4_status_string(-2) == b"NVFP4_ERR_UNSUPPORTED"
    assert lib.nvfp4_status_string(-3) == b"NVFP4_ERR_HIP"
    assert lib.nvfp4_status_string(7) == b"NVFP4_UNKNOWN_STATUS"
    assert re.fullmatch(rb"\d+\.\d+\.\d+", lib.nvfp4_version())


def test_workspace_bytes():
    assert nv.nvfp4_quantize_workspace_bytes(0, 16) == 0
    assert nv.nvfp4_quantize_workspace_bytes(16, 0) == 0
    assert nv.nvfp4_quantize_workspace_bytes(1, 16) == 4
    w = nv.nvfp4_quantize_workspace_bytes(4096, 8192)
    assert 4 <= w <= 4096 and w % 4 == 0


def _q(**kw):
    args = dict(x=P16, x_dtype=nv.NVFP4_BF16, rows=4, cols=32, ld_x=32, q=P16, s=P16,
                global_scale=P16, flags=0, workspace=P16, workspace_bytes=1024)
    args.update(kw)
    lib = nv.load()
    return lib.nvfp4_quantize(args["x"], args["x_dtype"], args["rows"], args["cols"],
                              args["ld_x"], args["q"], args["s"], args["global_scale"],
                              args["flags"], args["workspace"], args["workspace_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cols=24), nv.NVFP4_ERR_INVALID_ARG),
    (dict(rows=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x_dtype=5), nv.NVFP4_ERR_INVALID_ARG),
    (dict(flags=2), nv.NVFP4_ERR_INVALID_ARG),
    (dict(global_scale=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(q=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(s=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(ld_x=16), nv.NVFP4_ERR_INVALID_ARG),
    (dict(workspace=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(workspace_bytes=0), nv.NVFP4_ERR_INVALID_ARG),
    (dict(workspace=ctypes.c_void_p(0x10002)), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=P8), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(ld_x=36), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(q=P4), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=0), nv.NVFP4_OK),
    (dict(cols=0, ld_x=0), nv.NVFP4_OK),
])
def test_quantize_argument_checks(kw, status):
    assert _q(**kw) == status


def _g(**kw):
    args = dict(M=8, N=8, K=128, a_q=P16, a_s=P16, a_g=P16, b_q=P16, b_s=P16, b_g=P16,
                y=P16, y_dtype=nv.NVFP4_BF16, ld_y=8)
    args.update(kw)
    return nv.load().nvfp4_gemm(*[args[k] for k in ("M", "N", "K", "a_q", "a_s", "a_g", "b_q",
                                                    "b_s", "b_g", "y", "y_dtype", "ld_y")],
                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=24), nv.NVFP4_ERR_INVALID_ARG),
    (dict(M=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(N=-3), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_dtype=2), nv.NVFP4_ERR_INVALID_ARG),
    (dict(ld_y=7), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(a_q=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(b_s=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(a_g=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(b_g=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(K=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(M=0), nv.NVFP4_OK),
    (dict(N=0, ld_y=0), nv.NVFP4_OK),
])
def test_gemm_argument_checks(kw, status):
    assert _g(**kw) == status


def _gg(**kw):
    args = dict(G=4, m_offsets=P16, total_m=8, N=8, K=128, a_q=P16, a_s=P16, a_g=P16,
                b_q=P16, b_s=P16, b_g=P16, y=P16, y_dtype=nv.NVFP4_BF16, ld_y=8)
    args.update(kw)
    order = ("G", "m_offsets", "total_m", "N", "K", "a_q", "a_s", "a_g", "b_q", "b_s", "b_g",
             "y", "y_dtype", "ld_y")
    return nv.load().nvfp4_grouped_gemm(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=40), nv.NVFP4_ERR_INVALID_ARG),
    (dict(G=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(G=0), nv.NVFP4_ERR_INVALID_ARG),
    (dict(m_offsets=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(ld_y=4), nv.NVFP4_ERR_INVALID_ARG),
    (dict(b_q=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_dtype=9), nv.NVFP4_ERR_INVALID_ARG),
    (dict(total_m=0), nv.NVFP4_OK),
    (dict(G=0, total_m=0), nv.NVFP4_OK),
    (dict(N=0, ld_y=0), nv.NVFP4_OK),
])
def test_grouped_argument_checks(kw, status):
    assert _gg(**kw) == status


def _ggx(**kw):
    args = dict(G=4, m_offsets=P16, row_index=P16, total_m=8, a_rows=5, N=8, K=128, a_q=P16,
                a_s=P16, a_g=P16, b_q=P16, b_s=P16, b_g=P16, y=P16, y_dtype=nv.NVFP4_BF16, ld_y=8)
    args.update(kw)
    order = ("G", "m_offsets", "row_index", "total_m", "a_rows", "N", "K", "a_q", "a_s", "a_g",
             "b_q", "b_s", "b_g", "y", "y_dtype", "ld_y")
    return nv.load().nvfp4_grouped_gemm_gather(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(row_index=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(a_rows=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(K=40), nv.NVFP4_ERR_INVALID_ARG),
    (dict(G=0), nv.NVFP4_ERR_INVALID_ARG),
    (dict(m_offsets=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(a_q=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(a_rows=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(total_m=0, row_index=NULL), nv.NVFP4_OK),
    (dict(N=0, ld_y=0), nv.NVFP4_OK),
])
def test_grouped_gather_argument_checks(kw, status):
    assert _ggx(**kw) == status


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import nvfp4_block_scaled_gemm_amd._lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        L.load()


def _gq(**kw):
    args = dict(M=8, N=32, K=128, a_q=P16, a_s=P16, a_g=P16, b_q=P16, b_s=P16, b_g=P16,
                y_q=P16, y_s=P16, y_g=P16)
    args.update(kw)
    order = ("M", "N", "K", "a_q", "a_s", "a_g", "b_q", "b_s", "b_g", "y_q", "y_s", "y_g")
    return nv.load().nvfp4_gemm_nvfp4_out(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=40), nv.NVFP4_ERR_INVALID_ARG),          # blocks of 16 output columns
    (dict(K=40), nv.NVFP4_ERR_INVALID_ARG),
    (dict(M=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_g=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_q=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_s=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(b_s=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_q=P4), nv.NVFP4_ERR_UNSUPPORTED),        # q rows are written 8 bytes at a time
    (dict(M=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(M=0, y_q=NULL, y_s=NULL), nv.NVFP4_OK),
    (dict(N=0), nv.NVFP4_OK),
])
def test_gemm_nvfp4_out_argument_checks(kw, status):
    assert _gq(**kw) == status


def _packed_cpu(rows, K, n_g=1):
    return (torch.zeros((rows, K // 2), dtype=torch.uint8),
            torch.zeros((rows, K // 16), dtype=torch.uint8),
            torch.ones(n_g, dtype=torch.float32))


@pytest.mark.parametrize("case", ["y_dtype", "y_shape", "a_noncontig", "b_scale_shape",
                                  "g_dtype", "out_dtype", "cpu_tensors"])
def test_binding_rejects_mismatched_tensors(case):
    """The tensor wrappers check what the C ABI cannot see (dtypes, shapes,
    packing, device) and raise before any library call or GPU work."""
    M, N, K = 4, 32, 64
    a, b = _packed_cpu(M, K), _packed_cpu(N, K)
    kw = {}
    if case == "y_dtype":
        kw = dict(out_dtype="f32", y=torch.empty((M, N), dtype=torch.bfloat16))
    elif case == "y_shape":
        kw = dict(y=torch.empty((M, N + 1), dtype=torch.bfloat16))
    elif case == "a_noncontig":
        wide = torch.zeros((M, K), dtype=torch.uint8)
        a = (wide[:, : K // 2], a[1], a[2])
    elif case == "b_scale_shape":
        b = (b[0], torch.zeros((N, K // 8), dtype=torch.uint8), b[2])
    elif case == "g_dtype":
        a = (a[0], a[1], torch.ones(1, dtype=torch.float64))
    elif case == "out_dtype":
        kw = dict(out_dtype="fp8")
    with pytest.raises(ValueError):
        nv.nvfp4_gemm(a, b, **kw)


def test_binding_rejects_mismatched_quantize_and_grouped_tensors():
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(torch.zeros((4, 32), dtype=torch.float16))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(torch.zeros((4, 40), dtype=torch.float32))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(torch.zeros((4, 32)), out=_packed_cpu(4, 64))
    G, N, K, total = 3, 16, 64, 10
    bq = torch.zeros((G, N, K // 2), dtype=torch.uint8)
    bs = torch.zeros((G, N, K // 16), dtype=torch.uint8)
    b = (bq, bs, torch.ones(G))
    a = _packed_cpu(total, K)
    with pytest.raises(ValueError):   # int64 offsets
        nv.nvfp4_grouped_gemm(torch.zeros(G + 1, dtype=torch.int64), total, a, b)
    with pytest.raises(ValueError):   # one global scale for three experts
        nv.nvfp4_grouped_gemm(torch.zeros(G + 1, dtype=torch.int32), total, a, (bq, bs, torch.ones(1)))
    with pytest.raises(ValueError):   # CPU tensors
        nv.nvfp4_grouped_gemm(torch.zeros(G + 1, dtype=torch.int32), total, a, b)


def test_output_buffer_checks_on_host():
    """The binding's output check (host tensors stand in for GPU buffers:
    both report device -1 here)."""
    import nvfp4_block_scaled_gemm_amd._lib as L
    assert L._out(torch.empty((4, 8), dtype=torch.bfloat16), 4, 8, torch.bfloat16, -1) == 8
    wide = torch.empty((4, 16), dtype=torch.bfloat16)[:, :8]        # row stride 16
    assert L._out(wide, 4, 8, torch.bfloat16, -1) == 16
    for bad in (torch.empty(32, dtype=torch.bfloat16), torch.empty((4, 8)),
                torch.empty((8, 4), dtype=torch.bfloat16).t()):
        with pytest.raises(ValueError):
            L._out(bad, 4, 8, torch.bfloat16, -1)
    with pytest.raises(ValueError):                                # another device
        L._out(torch.empty((4, 8), dtype=torch.bfloat16), 4, 8, torch.bfloat16, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(cols=24), nv.NVFP4_ERR_INVALID_ARG),
    (dict(rows=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x_dtype=5), nv.NVFP4_ERR_INVALID_ARG),
    (dict(flags=2), nv.NVFP4_ERR_INVALID_ARG),
    (dict(global_scale=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(ld_x=16), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=P8), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(q=P4), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=0), nv.NVFP4_OK),
])
def test_quantize_noalloc_validation(kw, status):
    """The no-allocation quantiser validates like nvfp4_quantize (no
    workspace arguments) and touches nothing on an invalid call."""
    args = dict(x=P16, x_dtype=nv.NVFP4_BF16, rows=4, cols=32, ld_x=32, q=P16, s=P16,
                global_scale=P16, flags=0)
    args.update(kw)
    st = nv.load().nvfp4_quantize_noalloc(args["x"], args["x_dtype"], args["rows"], args["cols"],
                                          args["ld_x"], args["q"], args["s"],
                                          args["global_scale"], args["flags"], None)
    assert st == status


def _gp(**kw):
    args = dict(G=4, m_offsets=0x10000, row_index=None, total_m=8, a_rows=0, N=8, K=128,
                a_q=0x10000, a_s=0x10000, a_g=0x10000, b_q=0x10000, b_s=0x10000, b_g=0x10000,
                y=0x10000, y_dtype=nv.NVFP4_BF16, ld_y=8)
    args.update(kw)
    return nv.GroupedProblem(**args)


def _multi(probs, count=None):
    arr = (nv.GroupedProblem * max(len(probs), 1))(*probs)
    return nv.load().nvfp4_grouped_gemm_multi(len(probs) if count is None else count, arr, None)


def test_grouped_problem_struct_layout():
    """The ctypes mirror of nvfp4_grouped_problem has the C layout (x86-64:
    int32 G padded to 8, then pointers and int64s, int y_dtype padded)."""
    assert ctypes.sizeof(nv.GroupedProblem) == 128
    assert nv.GroupedProblem.m_offsets.offset == 8
    assert nv.GroupedProblem.y_dtype.offset == 112
    assert nv.GroupedProblem.ld_y.offset == 120


@pytest.mark.parametrize("probs,count,status", [
    ([], None, nv.NVFP4_OK),
    ([_gp()], -1, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp()] * 5, None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(K=40)], None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(total_m=0), _gp(K=40)], None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(total_m=0), _gp(m_offsets=None)], None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(total_m=0), _gp(a_rows=5)], None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(row_index=0x10000, a_rows=-1)], None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(row_index=0x10000, a_rows=1 << 31)], None, nv.NVFP4_ERR_UNSUPPORTED),
    ([_gp(total_m=0), _gp(N=0, ld_y=0), _gp(G=0, total_m=0)], None, nv.NVFP4_OK),
    ([_gp(total_m=0), _gp(ld_y=4)], None, nv.NVFP4_ERR_INVALID_ARG),
    ([_gp(total_m=0), _gp(y_dtype=7)], None, nv.NVFP4_ERR_INVALID_ARG),
])
def test_grouped_multi_argument_checks(probs, count, status):
    """Every problem is validated before anything is enqueued: an invalid
    one anywhere in the list fails the call; empty problems are skipped."""
    assert _multi(probs, count) == status


def test_grouped_multi_null_problem_list():
    assert nv.load().nvfp4_grouped_gemm_multi(1, None, None) == nv.NVFP4_ERR_INVALID_ARG
    assert nv.load().nvfp4_grouped_gemm_multi(0, None, None) == nv.NVFP4_OK


def _mxq(**kw):
    args = dict(x=P16, x_dtype=nv.NVFP4_BF16, rows=4, cols=64, ld_x=64, q=P16, s=P16)
    args.update(kw)
    return nv.load().nvfp4_mxfp4_quantize(args["x"], args["x_dtype"], args["rows"], args["cols"],
                                          args["ld_x"], args["q"], args["s"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cols=48), nv.NVFP4_ERR_INVALID_ARG),
    (dict(rows=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x_dtype=5), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(s=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(ld_x=32), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=P8), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(q=P8), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(ld_x=68), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=0), nv.NVFP4_OK),
    (dict(cols=0, ld_x=0), nv.NVFP4_OK),
])
def test_mxfp4_quantize_argument_checks(kw, status):
    assert _mxq(**kw) == status


def _mxg(**kw):
    args = dict(M=4, N=8, K=128, a_q=P16, a_s=P16, b_q=P16, b_s=P16, y=P16,
                y_dtype=nv.NVFP4_BF16, ld_y=8)
    args.update(kw)
    order = ("M", "N", "K", "a_q", "a_s", "b_q", "b_s", "y", "y_dtype", "ld_y")
    return nv.load().nvfp4_mxfp4_gemm(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=48), nv.NVFP4_ERR_INVALID_ARG),
    (dict(M=-1), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y_dtype=2), nv.NVFP4_ERR_INVALID_ARG),
    (dict(ld_y=4), nv.NVFP4_ERR_INVALID_ARG),
    (dict(y=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(b_s=NULL), nv.NVFP4_ERR_INVALID_ARG),
    (dict(N=1 << 31, ld_y=1 << 31), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(M=0), nv.NVFP4_OK),
    (dict(N=0, ld_y=0), nv.NVFP4_OK),
])
def test_mxfp4_gemm_argument_checks(kw, status):
    assert _mxg(**kw) == status


def test_mxfp4_binding_rejects_mismatched_tensors():
    q = torch.zeros((4, 32), dtype=torch.uint8)
    s = torch.zeros((4, 4), dtype=torch.uint8)   # K = 64 needs 2 scale bytes per row
    with pytest.raises(ValueError):
        nv.nvfp4_mxfp4_gemm((q, s), (q, s))
    with pytest.raises(ValueError):
        nv.nvfp4_mxfp4_quantize(torch.zeros((4, 48), dtype=torch.bfloat16))
