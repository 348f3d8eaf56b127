"""ctypes binding of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch supplies device memory (``data_ptr``) and the
current HIP stream.  If the library has not been built, loading raises;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERR_INVALID_ARG = -1
NVFP4_ERR_UNSUPPORTED = -2
NVFP4_ERR_HIP = -3
NVFP4_F32 = 0
NVFP4_BF16 = 1
NVFP4_GLOBAL_SCALE_GIVEN = 1

EXPORTED = ("nvfp4_status_string", "nvfp4_version", "nvfp4_quantize_workspace_bytes",
            "nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_nvfp4_out", "nvfp4_grouped_gemm",
            "nvfp4_grouped_gemm_gather")

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libnvfp4.so once; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; run `python -m "
                          "nvfp4_block_scaled_gemm_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.nvfp4_status_string.argtypes = [ctypes.c_int]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_version.argtypes = []
    lib.nvfp4_version.restype = ctypes.c_char_p
    lib.nvfp4_quantize_workspace_bytes.argtypes = [i64, i64]
    lib.nvfp4_quantize_workspace_bytes.restype = sz
    lib.nvfp4_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, p, ctypes.c_uint,
                                   p, sz, p]
    lib.nvfp4_quantize.restype = ctypes.c_int
    lib.nvfp4_gemm.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, ctypes.c_int, i64, p]
    lib.nvfp4_gemm.restype = ctypes.c_int
    lib.nvfp4_gemm_nvfp4_out.argtypes = [i64, i64, i64, p, p, p, p, p, p, p, p, p, p]
    lib.nvfp4_gemm_nvfp4_out.restype = ctypes.c_int
    lib.nvfp4_grouped_gemm.argtypes = [i32, p, i64, i64, i64, p, p, p, p, p, p, p,
                                       ctypes.c_int, i64, p]
    lib.nvfp4_grouped_gemm.restype = ctypes.c_int
    lib.nvfp4_grouped_gemm_gather.argtypes = [i32, p, p, i64, i64, i64, i64, p, p, p, p, p, p,
                                              p, ctypes.c_int, i64, p]
    lib.nvfp4_grouped_gemm_gather.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != NVFP4_OK:
        msg = load().nvfp4_status_string(status).decode()
        raise Nvfp4Error(fn, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DT_IN = {torch.float32: NVFP4_F32, torch.bfloat16: NVFP4_BF16}
_DT_OUT = {"f32": (NVFP4_F32, torch.float32), "bf16": (NVFP4_BF16, torch.bfloat16)}


# The library reads packed operands as row-major [rows, K/2] and [rows, K/16]
# bytes and writes outputs of the dtype it is told; these checks keep a
# mismatched tensor from reaching it (they raise before any GPU work).
def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_gpu(dev, *ts):
    for t in ts:
        _need(t.is_cuda and t.device == dev, f"tensors must all be on {dev}")


def _packed(t3, rows: int, K: int, what: str, n_g: int = 1):
    """(q, s, g) of a packed operand [.., rows, K]: uint8 q [.., rows, K/2] and
    s [.., rows, K/16], contiguous; fp32 g with n_g elements."""
    q, s, g = t3
    lead = tuple(q.shape[:-2])
    _need(q.dtype == torch.uint8 and s.dtype == torch.uint8, f"{what}: q and s must be uint8")
    _need(tuple(q.shape) == (*lead, rows, K // 2) and tuple(s.shape) == (*lead, rows, K // 16),
          f"{what}: q {tuple(q.shape)} and s {tuple(s.shape)} do not pack [{rows}, {K}]")
    _need(q.is_contiguous() and s.is_contiguous(), f"{what}: q and s must be contiguous")
    _need(g.dtype == torch.float32 and g.numel() == n_g and g.is_contiguous(),
          f"{what}: g must be {n_g} contiguous fp32 value(s)")


def _out(y, rows: int, cols: int, dtype, what: str = "y"):
    _need(y.dtype == dtype, f"{what}: dtype {y.dtype}, expected {dtype}")
    _need(y.dim() == 2 and tuple(y.shape) == (rows, cols), f"{what}: shape {tuple(y.shape)}, "
          f"expected ({rows}, {cols})")
    _need(y.stride(1) == 1 or cols <= 1, f"{what}: rows must have unit column stride")


# --------------------------------------------------------------------------
# raw entry points (same names and arguments as the C ABI)
# --------------------------------------------------------------------------

def nvfp4_quantize_workspace_bytes(rows: int, cols: int) -> int:
    return int(load().nvfp4_quantize_workspace_bytes(rows, cols))


def nvfp4_quantize_raw(x, x_dtype, rows, cols, ld_x, q, s, global_scale, flags,
                       workspace, workspace_bytes, stream=None) -> int:
    return load().nvfp4_quantize(x, x_dtype, rows, cols, ld_x, q, s, global_scale, flags,
                                 workspace, workspace_bytes, _stream(stream))


def nvfp4_gemm_raw(M, N, K, a_q, a_s, a_g, b_q, b_s, b_g, y, y_dtype, ld_y,
                   stream=None) -> int:
    return load().nvfp4_gemm(M, N, K, a_q, a_s, a_g, b_q, b_s, b_g, y, y_dtype, ld_y,
                             _stream(stream))


def nvfp4_gemm_nvfp4_out_raw(M, N, K, a_q, a_s, a_g, b_q, b_s, b_g, y_q, y_s, y_g,
                             stream=None) -> int:
    return load().nvfp4_gemm_nvfp4_out(M, N, K, a_q, a_s, a_g, b_q, b_s, b_g, y_q, y_s, y_g,
                                       _stream(stream))


def nvfp4_grouped_gemm_raw(G, m_offsets, total_m, N, K, a_q, a_s, a_g, b_q, b_s, b_g, y,
                           y_dtype, ld_y, stream=None) -> int:
    return load().nvfp4_grouped_gemm(G, m_offsets, total_m, N, K, a_q, a_s, a_g, b_q, b_s,
                                     b_g, y, y_dtype, ld_y, _stream(stream))


def nvfp4_grouped_gemm_gather_raw(G, m_offsets, row_index, total_m, a_rows, N, K, a_q, a_s,
                                  a_g, b_q, b_s, b_g, y, y_dtype, ld_y, stream=None) -> int:
    return load().nvfp4_grouped_gemm_gather(G, m_offsets, row_index, total_m, a_rows, N, K,
                                            a_q, a_s, a_g, b_q, b_s, b_g, y, y_dtype, ld_y,
                                            _stream(stream))


# --------------------------------------------------------------------------
# tensor-level wrappers (allocate outputs with torch, then call the C ABI)
# --------------------------------------------------------------------------

def nvfp4_quantize(x: torch.Tensor, global_scale: torch.Tensor | None = None,
                   out=None, workspace: torch.Tensor | None = None, stream=None):
    """x [rows, cols] fp32/bf16 on the GPU -> (q uint8 [rows, cols/2],
    s uint8 [rows, cols/16], g fp32 [1]).  ``global_scale`` (device fp32 [1])
    switches to the static-scale path; ``out`` = (q, s, g) reuses buffers."""
    _need(x.dim() == 2 and x.dtype in _DT_IN, "x: 2-D fp32 or bf16")
    _need(x.stride(1) == 1 or x.shape[1] <= 1, "x: rows must have unit column stride")
    rows, cols = x.shape
    _need(cols % 16 == 0, "x: columns must be a multiple of 16")
    dev = x.device
    if out is None:
        _on_gpu(dev, x)
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        q, s, g = out
        _packed((q, s, g), rows, cols, "out")
    if global_scale is not None:
        _need(global_scale.dtype == torch.float32 and global_scale.numel() == 1,
              "global_scale: one fp32 value")
        _on_gpu(dev, global_scale)
    if workspace is not None:
        _on_gpu(dev, workspace)
    _on_gpu(dev, x, q, s, g)
    flags = 0
    if global_scale is not None:
        g.copy_(global_scale.reshape(1))
        flags = NVFP4_GLOBAL_SCALE_GIVEN
    ws_bytes = nvfp4_quantize_workspace_bytes(rows, cols)
    if workspace is None and flags == 0:
        workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=dev)
    st = nvfp4_quantize_raw(_ptr(x), _DT_IN[x.dtype], rows, cols, x.stride(0), _ptr(q), _ptr(s),
                            _ptr(g), flags, _ptr(workspace),
                            0 if workspace is None else workspace.numel() * workspace.element_size(),
                            stream)
    _check("nvfp4_quantize", st)
    return q, s, g


def nvfp4_gemm(a, b, out_dtype: str = "bf16", y: torch.Tensor | None = None, stream=None):
    """a = (q, s, g) of x [M, K]; b = (q, s, g) of W [N, K] -> y [M, N]."""
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    _need(a_q.dim() == 2 and b_q.dim() == 2, "a and b: 2-D packed operands")
    M, N, K = a_q.shape[0], b_q.shape[0], a_q.shape[1] * 2
    _packed(a, M, K, "a")
    _packed(b, N, K, "b")
    _need(out_dtype in _DT_OUT, f"out_dtype: one of {sorted(_DT_OUT)}")
    code, tdt = _DT_OUT[out_dtype]
    if y is None:
        y = torch.empty((M, N), dtype=tdt, device=a_q.device)
    _out(y, M, N, tdt)
    _on_gpu(a_q.device, a_q, a_s, a_g, b_q, b_s, b_g, y)
    st = nvfp4_gemm_raw(M, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q), _ptr(b_s),
                        _ptr(b_g), _ptr(y), code, y.stride(0), stream)
    _check("nvfp4_gemm", st)
    return y


def nvfp4_gemm_nvfp4_out(a, b, y_g: torch.Tensor, out=None, stream=None):
    """a = (q, s, g) of x [M, K], b = (q, s, g) of W [N, K]; y_g = the output's
    static global scale (fp32 [1], GPU) -> (q [M, N/2], s [M, N/16], y_g): y
    quantised in the GEMM's epilogue.  ``out`` = (q, s) reuses buffers."""
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    _need(a_q.dim() == 2 and b_q.dim() == 2, "a and b: 2-D packed operands")
    M, N, K = a_q.shape[0], b_q.shape[0], a_q.shape[1] * 2
    _packed(a, M, K, "a")
    _packed(b, N, K, "b")
    _need(N % 16 == 0, "the output's columns (rows of b) must be a multiple of 16")
    if out is None:
        q = torch.empty((M, N // 2), dtype=torch.uint8, device=a_q.device)
        s = torch.empty((M, N // 16), dtype=torch.uint8, device=a_q.device)
    else:
        q, s = out
    _packed((q, s, y_g), M, N, "out")
    _on_gpu(a_q.device, a_q, a_s, a_g, b_q, b_s, b_g, q, s, y_g)
    st = nvfp4_gemm_nvfp4_out_raw(M, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q),
                                  _ptr(b_s), _ptr(b_g), _ptr(q), _ptr(s), _ptr(y_g), stream)
    _check("nvfp4_gemm_nvfp4_out", st)
    return q, s, y_g


def nvfp4_grouped_gemm(m_offsets: torch.Tensor, total_m: int, a, b, out_dtype: str = "bf16",
                       y: torch.Tensor | None = None, stream=None,
                       row_index: torch.Tensor | None = None):
    """m_offsets int32 [G+1] (GPU); a = (q [total_m, K/2], s, g [1]);
    b = (q [G, N, K/2], s [G, N, K/16], g [G]) -> y [total_m, N].
    With row_index (int32 [total_m], GPU), grouped row r reads row
    row_index[r] of a = (q [a_rows, K/2], s, g) instead (no gathered copy)."""
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    _need(b_q.dim() == 3 and a_q.dim() == 2, "b: [G, N, K/2] packed experts; a: 2-D packed rows")
    G, N = b_q.shape[0], b_q.shape[1]
    K = b_q.shape[2] * 2
    _packed(b, N, K, "b", n_g=G)
    _packed(a, a_q.shape[0] if row_index is not None else total_m, K, "a")
    _need(m_offsets.dtype == torch.int32 and m_offsets.numel() == G + 1
          and m_offsets.is_contiguous(), "m_offsets: G + 1 contiguous int32")
    _need(out_dtype in _DT_OUT, f"out_dtype: one of {sorted(_DT_OUT)}")
    code, tdt = _DT_OUT[out_dtype]
    if y is None:
        y = torch.empty((total_m, N), dtype=tdt, device=b_q.device)
    _out(y, total_m, N, tdt)
    _on_gpu(b_q.device, a_q, a_s, a_g, b_q, b_s, b_g, m_offsets, y)
    if row_index is None:
        st = nvfp4_grouped_gemm_raw(G, _ptr(m_offsets), total_m, N, K, _ptr(a_q), _ptr(a_s),
                                    _ptr(a_g), _ptr(b_q), _ptr(b_s), _ptr(b_g), _ptr(y), code,
                                    y.stride(0), stream)
        _check("nvfp4_grouped_gemm", st)
        return y
    _need(row_index.dtype == torch.int32 and row_index.numel() == total_m
          and row_index.is_contiguous(), "row_index: total_m contiguous int32")
    _on_gpu(b_q.device, row_index)
    st = nvfp4_grouped_gemm_gather_raw(G, _ptr(m_offsets), _ptr(row_index), total_m,
                                       a_q.shape[0], N, K, _ptr(a_q), _ptr(a_s), _ptr(a_g),
                                       _ptr(b_q), _ptr(b_s), _ptr(b_g), _ptr(y), code,
                                       y.stride(0), stream)
    _check("nvfp4_grouped_gemm_gather", st)
    return y
