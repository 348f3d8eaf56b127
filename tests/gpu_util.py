"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
from oracle import global_scale_ref, quantize_ref


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg: str):
    """Print a progress line naming the case before a GPU step."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def np_(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def oracle_quantize(x_cpu: torch.Tensor, global_scale=None):
    """Oracle quantisation of a CPU tensor (fp32 or bf16; bf16 widens exactly)."""
    return quantize_ref(np_(x_cpu), global_scale=global_scale)


def oracle_global_scale(x_cpu: torch.Tensor) -> np.float32:
    """The oracle's global scale of a whole CPU tensor (bf16 widens exactly)."""
    return global_scale_ref(np_(x_cpu))


def to_gpu(q, s, g):
    dev = torch.device("cuda")
    return (torch.from_numpy(np.ascontiguousarray(q)).to(dev),
            torch.from_numpy(np.ascontiguousarray(s)).to(dev),
            torch.tensor([float(g)], dtype=torch.float32, device=dev))


def assert_bytes_equal(gpu_q, gpu_s, gpu_g, ref_q, ref_s, ref_g, rows=None):
    gq, gs = np_(gpu_q), np_(gpu_s)
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    assert np.float32(np_(gpu_g)[0]).view(np.uint32) == np.float32(ref_g).view(np.uint32), \
        (np_(gpu_g)[0], ref_g)
    bad_s = np.argwhere(gs != ref_s)
    assert bad_s.size == 0, f"scale bytes differ at {bad_s[:5].tolist()}: " \
        f"gpu {gs[tuple(bad_s[0])]:#x} ref {ref_s[tuple(bad_s[0])]:#x}"
    bad_q = np.argwhere(gq != ref_q)
    assert bad_q.size == 0, f"packed bytes differ at {bad_q[:5].tolist()}: " \
        f"gpu {gq[tuple(bad_q[0])]:#x} ref {ref_q[tuple(bad_q[0])]:#x}"
