"""ctypes binding of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch supplies device memory (``data_ptr``) and the
current HIP stream.  If the library has not been built, loading raises;
there is no fallback implementation.
"""
from __future__ import annotations

import contextlib
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
            "nvfp4_quantize", "nvfp4_quantize_noalloc", "nvfp4_gemm", "nvfp4_gemm_nvfp4_out", "nvfp4_grouped_gemm",
            "nvfp4_grouped_gemm_gather", "nvfp4_grouped_gemm_multi", "nvfp4_mxfp4_quantize",
            "nvfp4_mxfp4_gemm")
NVFP4_GROUPED_MAX_PROBLEMS = 4

_lib = None


class GroupedProblem(ctypes.Structure):
    """nvfp4_grouped_problem of include/nvfp4.h (one grouped GEMM)."""
    _fields_ = [("G", ctypes.c_int32), ("m_offsets", ctypes.c_void_p),
                ("row_index", ctypes.c_void_p), ("total_m", ctypes.c_int64),
                ("a_rows", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_q", ctypes.c_void_p), ("a_s", ctypes.c_void_p), ("a_g", ctypes.c_void_p),
                ("b_q", ctypes.c_void_p), ("b_s", ctypes.c_void_p), ("b_g", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int), ("ld_y", ctypes.c_int64)]


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
    lib.nvfp4_quantize_noalloc.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, p, ctypes.c_uint,
                                           p]
    lib.nvfp4_quantize_noalloc.restype = ctypes.c_int
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
    lib.nvfp4_grouped_gemm_multi.argtypes = [i32, ctypes.POINTER(GroupedProblem), p]
    lib.nvfp4_grouped_gemm_multi.restype = ctypes.c_int
    lib.nvfp4_mxfp4_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, p]
    lib.nvfp4_mxfp4_quantize.restype = ctypes.c_int
    lib.nvfp4_mxfp4_gemm.argtypes = [i64, i64, i64, p, p, p, p, p, ctypes.c_int, i64, p]
    lib.nvfp4_mxfp4_gemm.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != NVFP4_OK:
        msg = load().nvfp4_status_string(status).decode()
        raise Nvfp4Error(fn, status, msg)


def _ptr(t):
    # the pointer arguments are declared c_void_p, so a plain int is passed
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream=None, dev: int | None = None):
    """HIP stream handle: ``stream`` (a torch stream or a raw handle), else the
    current stream of device ``dev`` (default: the current device)."""
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if dev is None:
        dev = torch.cuda.current_device()
    if _raw_stream is not None:
        return _raw_stream(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _on_stream(stream, dev: int):
    """Context in which the wrapper's own torch work (output allocations, the
    static-scale copy, its internal workspace) is ordered on the same stream
    as the library call: ``stream`` when given (a torch stream or a raw
    handle), else nothing to change (the current stream is used by both)."""
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=dev)
    return torch.cuda.stream(stream)


_DT_IN = {torch.float32: NVFP4_F32, torch.bfloat16: NVFP4_BF16}
_DT_OUT = {"f32": (NVFP4_F32, torch.float32), "bf16": (NVFP4_BF16, torch.bfloat16)}


# The library reads packed operands as row-major [rows, K/2] and [rows, K/16]
# bytes and writes outputs of the dtype it is told; these checks keep a
# mismatched tensor from reaching it (they raise before any GPU work).  A
# packed operand is checked once, when it becomes a ``Packed``, so that the
# per-call cost stays small next to a few-microsecond decode GEMM.
def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


class Packed(tuple):
    """(q, s, g) of an NVFP4 tensor [rows, K], or of G expert weights
    [G, rows, K]: uint8 q [.., rows, K/2] and s [.., rows, K/16], both
    contiguous, and fp32 g (one value, or one per expert), all on one GPU.
    Checked when made; nvfp4_quantize returns one.  Changing the tensors'
    shapes in place afterwards is not supported."""

    def __new__(cls, ts, _trusted=None):
        q, s, g = ts
        self = super().__new__(cls, (q, s, g))
        if _trusted is not None:
            self.lead, self.rows, self.K, self.dev = _trusted
            return self
        _need(q.dim() >= 2, "q: at least 2-D")
        lead = tuple(q.shape[:-2])
        rows, K = q.shape[-2], q.shape[-1] * 2
        _need(q.dtype == torch.uint8 and s.dtype == torch.uint8, "q and s must be uint8")
        _need(tuple(s.shape) == (*lead, rows, K // 16) and K % 16 == 0,
              f"q {tuple(q.shape)} and s {tuple(s.shape)} do not pack [{rows}, {K}]")
        _need(q.is_contiguous() and s.is_contiguous(), "q and s must be contiguous")
        n_g = lead[0] if len(lead) == 1 else 1
        _need(len(lead) <= 1, "at most one leading (expert) dimension")
        _need(g.dtype == torch.float32 and g.numel() == n_g and g.is_contiguous(),
              f"g must be {n_g} contiguous fp32 value(s)")
        dev = q.get_device()
        _need(q.is_cuda and s.get_device() == dev and g.get_device() == dev,
              "q, s and g must be on one GPU")
        self.lead, self.rows, self.K, self.dev = lead, rows, K, dev
        return self


def _packed(t3) -> Packed:
    return t3 if type(t3) is Packed else Packed(t3)


def _out(y, rows: int, cols: int, dtype, dev: int, what: str = "y") -> int:
    """Checks an output [rows, cols] of ``dtype`` on GPU ``dev``; returns its
    row stride."""
    st = y.stride()
    if y.dtype == dtype and y.shape == (rows, cols) and (st[1] == 1 or cols <= 1) \
            and y.get_device() == dev:
        return st[0]
    _need(y.dtype == dtype, f"{what}: dtype {y.dtype}, expected {dtype}")
    _need(y.shape == (rows, cols), f"{what}: shape {tuple(y.shape)}, expected ({rows}, {cols})")
    _need(st[1] == 1 or cols <= 1, f"{what}: rows must have unit column stride")
    raise ValueError(f"{what}: must be on the operands' GPU")


def _on_dev(t, dev: int, what: str):
    _need(t.get_device() == dev, f"{what}: must be on the operands' GPU")


# --------------------------------------------------------------------------
# raw entry points (same names and arguments as the C ABI)
# --------------------------------------------------------------------------

def nvfp4_quantize_workspace_bytes(rows: int, cols: int) -> int:
    return int(load().nvfp4_quantize_workspace_bytes(rows, cols))


def nvfp4_quantize_raw(x, x_dtype, rows, cols, ld_x, q, s, global_scale, flags,
                       workspace, workspace_bytes, stream=None) -> int:
    return load().nvfp4_quantize(x, x_dtype, rows, cols, ld_x, q, s, global_scale, flags,
                                 workspace, workspace_bytes, _stream(stream))


def nvfp4_quantize_noalloc_raw(x, x_dtype, rows, cols, ld_x, q, s, global_scale, flags,
                               stream=None) -> int:
    return load().nvfp4_quantize_noalloc(x, x_dtype, rows, cols, ld_x, q, s, global_scale, flags,
                                         _stream(stream))


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
    _need(x.is_cuda, "x: must be on a GPU")
    with _on_stream(stream, x.get_device()):
        return _quantize(x, global_scale, out, workspace)


def _quantize(x, global_scale, out, workspace):
    rows, cols = x.shape
    dev = x.device
    di = x.get_device()
    if out is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
        res = Packed((q, s, g), _trusted=((), rows, cols, di))
    else:
        res = _packed(tuple(out))
        _need(not res.lead and res.rows == rows and res.K == cols and res.dev == di,
              f"out: does not pack x [{rows}, {cols}] on its GPU")
        q, s, g = res
    if global_scale is not None:
        _need(global_scale.dtype == torch.float32 and global_scale.numel() == 1,
              "global_scale: one fp32 value")
        _on_dev(global_scale, di, "global_scale")
    if workspace is not None:
        _on_dev(workspace, di, "workspace")
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
                            _stream(None, di))
    _check("nvfp4_quantize", st)
    return res


def nvfp4_gemm(a, b, out_dtype: str = "bf16", y: torch.Tensor | None = None, stream=None):
    """a = (q, s, g) of x [M, K]; b = (q, s, g) of W [N, K] -> y [M, N]."""
    if type(a) is not Packed:
        a = Packed(a)
    if type(b) is not Packed:
        b = Packed(b)
    if a.lead or b.lead or a.K != b.K or a.dev != b.dev:
        raise ValueError("a and b: 2-D packed operands with the same K on one GPU")
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    M, N, K = a.rows, b.rows, a.K
    _need(out_dtype in _DT_OUT, f"out_dtype: one of {sorted(_DT_OUT)}")
    code, tdt = _DT_OUT[out_dtype]
    if y is None:
        with _on_stream(stream, a.dev):
            y = torch.empty((M, N), dtype=tdt, device=a_q.device)
    ld_y = _out(y, M, N, tdt, a.dev)
    st = nvfp4_gemm_raw(M, N, K, a_q.data_ptr(), a_s.data_ptr(), a_g.data_ptr(), b_q.data_ptr(),
                        b_s.data_ptr(), b_g.data_ptr(), y.data_ptr(), code, ld_y,
                        _stream(stream, a.dev))
    _check("nvfp4_gemm", st)
    return y


def nvfp4_gemm_nvfp4_out(a, b, y_g: torch.Tensor, out=None, stream=None):
    """a = (q, s, g) of x [M, K], b = (q, s, g) of W [N, K]; y_g = the output's
    static global scale (fp32 [1], GPU) -> (q [M, N/2], s [M, N/16], y_g): y
    quantised in the GEMM's epilogue.  ``out`` = (q, s) reuses buffers."""
    a, b = _packed(a), _packed(b)
    _need(not a.lead and not b.lead and a.K == b.K and a.dev == b.dev,
          "a and b: 2-D packed operands with the same K on one GPU")
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    M, N, K = a.rows, b.rows, a.K
    _need(N % 16 == 0, "the output's columns (rows of b) must be a multiple of 16")
    if out is None:
        with _on_stream(stream, a.dev):
            q = torch.empty((M, N // 2), dtype=torch.uint8, device=a_q.device)
            s = torch.empty((M, N // 16), dtype=torch.uint8, device=a_q.device)
    else:
        q, s = out
    o = Packed((q, s, y_g))
    _need(not o.lead and o.rows == M and o.K == N and o.dev == a.dev,
          f"out: must pack the output [{M}, {N}] on the operands' GPU")
    st = nvfp4_gemm_nvfp4_out_raw(M, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q),
                                  _ptr(b_s), _ptr(b_g), _ptr(q), _ptr(s), _ptr(y_g),
                                  _stream(stream, a.dev))
    _check("nvfp4_gemm_nvfp4_out", st)
    return q, s, y_g


def _grouped_problem(m_offsets, total_m, a, b, out_dtype, y, stream, row_index):
    """Checks one grouped call's tensors; returns (GroupedProblem, y, dev)."""
    a, b = _packed(a), _packed(b)
    _need(len(b.lead) == 1 and not a.lead and a.K == b.K and a.dev == b.dev,
          "b: [G, N, K/2] packed experts and a: packed rows with the same K, on one GPU")
    _need(row_index is not None or a.rows == total_m, "a: total_m rows (or give row_index)")
    a_q, a_s, a_g = a
    b_q, b_s, b_g = b
    G, N, K = b.lead[0], b.rows, b.K
    _need(m_offsets.dtype == torch.int32 and m_offsets.numel() == G + 1
          and m_offsets.is_contiguous(), "m_offsets: G + 1 contiguous int32")
    _on_dev(m_offsets, b.dev, "m_offsets")
    _need(out_dtype in _DT_OUT, f"out_dtype: one of {sorted(_DT_OUT)}")
    code, tdt = _DT_OUT[out_dtype]
    if y is None:
        with _on_stream(stream, b.dev):
            y = torch.empty((total_m, N), dtype=tdt, device=b_q.device)
    ld_y = _out(y, total_m, N, tdt, b.dev)
    a_rows = 0
    if row_index is not None:
        _need(row_index.dtype == torch.int32 and row_index.numel() == total_m
              and row_index.is_contiguous(), "row_index: total_m contiguous int32")
        _on_dev(row_index, b.dev, "row_index")
        a_rows = a_q.shape[0]
    prob = GroupedProblem(G, _ptr(m_offsets), _ptr(row_index) if row_index is not None else None,
                          total_m, a_rows, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_g), _ptr(b_q),
                          _ptr(b_s), _ptr(b_g), _ptr(y), code, ld_y)
    return prob, y, b.dev


def nvfp4_grouped_gemm(m_offsets: torch.Tensor, total_m: int, a, b, out_dtype: str = "bf16",
                       y: torch.Tensor | None = None, stream=None,
                       row_index: torch.Tensor | None = None):
    """m_offsets int32 [G+1] (GPU); a = (q [total_m, K/2], s, g [1]);
    b = (q [G, N, K/2], s [G, N, K/16], g [G]) -> y [total_m, N].
    With row_index (int32 [total_m], GPU), grouped row r reads row
    row_index[r] of a = (q [a_rows, K/2], s, g) instead (no gathered copy)."""
    p, y, dev = _grouped_problem(m_offsets, total_m, a, b, out_dtype, y, stream, row_index)
    stream = _stream(stream, dev)
    if row_index is None:
        st = nvfp4_grouped_gemm_raw(p.G, p.m_offsets, total_m, p.N, p.K, p.a_q, p.a_s, p.a_g,
                                    p.b_q, p.b_s, p.b_g, p.y, p.y_dtype, p.ld_y, stream)
        _check("nvfp4_grouped_gemm", st)
        return y
    st = nvfp4_grouped_gemm_gather_raw(p.G, p.m_offsets, p.row_index, total_m, p.a_rows, p.N,
                                       p.K, p.a_q, p.a_s, p.a_g, p.b_q, p.b_s, p.b_g, p.y,
                                       p.y_dtype, p.ld_y, stream)
    _check("nvfp4_grouped_gemm_gather", st)
    return y


def nvfp4_grouped_gemm_multi_raw(problems, stream=None) -> int:
    """problems: a sequence of GroupedProblem (host structures)."""
    arr = (GroupedProblem * max(len(problems), 1))(*problems)
    return load().nvfp4_grouped_gemm_multi(len(problems), arr, _stream(stream))


def nvfp4_grouped_gemm_multi(calls, stream=None):
    """Several grouped GEMMs in one launch.  `calls` is a sequence (at most
    NVFP4_GROUPED_MAX_PROBLEMS) of dicts holding nvfp4_grouped_gemm's
    arguments (m_offsets, total_m, a, b and optionally out_dtype, y,
    row_index); returns their outputs, equal bit for bit to those of the
    separate calls."""
    _need(len(calls) <= NVFP4_GROUPED_MAX_PROBLEMS,
          f"at most {NVFP4_GROUPED_MAX_PROBLEMS} grouped problems per launch")
    probs, ys, devs = [], [], set()
    for c in calls:
        p, y, dev = _grouped_problem(c["m_offsets"], c["total_m"], c["a"], c["b"],
                                     c.get("out_dtype", "bf16"), c.get("y"), stream,
                                     c.get("row_index"))
        probs.append(p)
        ys.append(y)
        devs.add(dev)
    if not probs:
        return ys
    _need(len(devs) == 1, "all problems on one GPU")
    st = nvfp4_grouped_gemm_multi_raw(probs, _stream(stream, devs.pop()))
    _check("nvfp4_grouped_gemm_multi", st)
    return ys


# --------------------------------------------------------------------------
# MXFP4 variant (32-element blocks, E8M0 scales, no per-tensor scale)
# --------------------------------------------------------------------------

def nvfp4_mxfp4_quantize_raw(x, x_dtype, rows, cols, ld_x, q, s, stream=None) -> int:
    return load().nvfp4_mxfp4_quantize(x, x_dtype, rows, cols, ld_x, q, s, _stream(stream))


def nvfp4_mxfp4_gemm_raw(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype, ld_y, stream=None) -> int:
    return load().nvfp4_mxfp4_gemm(M, N, K, a_q, a_s, b_q, b_s, y, y_dtype, ld_y,
                                   _stream(stream))


def _mx_operand(t2, what: str):
    """(q uint8 [rows, K/2], s uint8 [rows, K/32]) on one GPU -> (rows, K, dev)."""
    q, s = t2
    _need(q.dim() == 2 and q.dtype == torch.uint8 and s.dtype == torch.uint8,
          f"{what}: q and s must be 2-D uint8")
    rows, K = q.shape[0], q.shape[1] * 2
    _need(tuple(s.shape) == (rows, K // 32) and K % 32 == 0,
          f"{what}: q {tuple(q.shape)} and s {tuple(s.shape)} do not pack [{rows}, {K}] in blocks of 32")
    _need(q.is_contiguous() and s.is_contiguous(), f"{what}: q and s must be contiguous")
    _need(q.is_cuda and s.get_device() == q.get_device(), f"{what}: q and s must be on one GPU")
    return rows, K, q.get_device()


def nvfp4_mxfp4_quantize(x: torch.Tensor, out=None, stream=None):
    """x [rows, cols] fp32/bf16 on the GPU (cols % 32 == 0) -> (q uint8
    [rows, cols/2], s uint8 [rows, cols/32]) in MXFP4; ``out`` reuses
    buffers."""
    _need(x.dim() == 2 and x.dtype in _DT_IN, "x: 2-D fp32 or bf16")
    _need(x.stride(1) == 1 or x.shape[1] <= 1, "x: rows must have unit column stride")
    _need(x.is_cuda, "x: must be on a GPU")
    rows, cols = x.shape
    _need(cols % 32 == 0, "x: columns must be a multiple of 32")
    di = x.get_device()
    with _on_stream(stream, di):
        if out is None:
            q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
            s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
        else:
            q, s = out
            r, K, dev = _mx_operand((q, s), "out")
            _need(r == rows and K == cols and dev == di, f"out: does not pack x [{rows}, {cols}] on its GPU")
        st = nvfp4_mxfp4_quantize_raw(_ptr(x), _DT_IN[x.dtype], rows, cols, x.stride(0), _ptr(q),
                                      _ptr(s), _stream(None, di))
    _check("nvfp4_mxfp4_quantize", st)
    return q, s


def nvfp4_mxfp4_gemm(a, b, out_dtype: str = "bf16", y: torch.Tensor | None = None, stream=None):
    """a = (q, s) of x [M, K]; b = (q, s) of W [N, K], both MXFP4 -> y [M, N]
    = x . W^T."""
    M, K, da = _mx_operand(a, "a")
    N, Kb, db = _mx_operand(b, "b")
    _need(K == Kb and da == db, "a and b: the same K, on one GPU")
    _need(out_dtype in _DT_OUT, f"out_dtype: one of {sorted(_DT_OUT)}")
    code, tdt = _DT_OUT[out_dtype]
    with _on_stream(stream, da):
        if y is None:
            y = torch.empty((M, N), dtype=tdt, device=a[0].device)
        ld_y = _out(y, M, N, tdt, da)
        st = nvfp4_mxfp4_gemm_raw(M, N, K, _ptr(a[0]), _ptr(a[1]), _ptr(b[0]), _ptr(b[1]), _ptr(y),
                                  code, ld_y, _stream(None, da))
    _check("nvfp4_mxfp4_gemm", st)
    return y
