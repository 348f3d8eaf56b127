"""Build libnvfp4.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m nvfp4_block_scaled_gemm_amd.build

Every source compiles to an object under ``_build/`` (in parallel), then one
shared library is linked next to this file.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")

ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of generated code (the device compile
# warns that the host target does not know the feature; that is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


# The decode-sized kernels (decode GEMMs, the quantiser's passes at a few
# rows, the 33-96 row GEMM) run for a few to ~20 us, so the latency of their
# first kernel-argument loads shows in the total: for them the compiler is
# asked to have the leading 14 argument dwords preloaded into SGPRs at wave
# launch (gfx950; the code object keeps a fallback entry that loads them when
# the firmware does not preload).
PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=14"]
EXTRA_FLAGS = {f: PRELOAD for f in ("gemm_decode_rows.hip", "gemm_decode_lds.hip", "gemm_skinny.hip", "quantize.hip")}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libnvfp4.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    # every host-side kernel stub must resolve: load the library once
    # (no GPU needed; a silently dropped template stub fails here)
    import ctypes
    try:
        ctypes.CDLL(tmp)
    except OSError as exc:
        raise RuntimeError(f"built library does not load: {exc}") from exc
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
