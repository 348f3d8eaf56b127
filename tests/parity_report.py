"""Parity report for the five workloads: the worst error of the GPU GEMM
against the fp64 oracle, as max |y - y_ref| / sum_k |x_k w_k| (fp32 output,
i.e. the accumulation before any bf16 rounding) and as a fraction of the
tolerance 1e-5 * sum_k |x_k w_k|, plus whether the quantised bytes match.

Not a test (pytest does not collect it); it prints one JSON line per
workload.  Run on a GPU from the repository root:

    python3 tests/parity_report.py

Samples follow the parity tests: the tiny workload in full; the linear layer
on 256 x 256 outputs; decode on 1024 columns; the MoE gate_up and down on
256 columns of experts 0, 97 and 255; the 16384^3 workload on 32 x 32
outputs (each over all of K).
"""
from __future__ import annotations

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import nvfp4_block_scaled_gemm_amd as nv  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import np_, oracle_global_scale, oracle_quantize  # noqa: E402
from oracle import gemm_ref  # noqa: E402


def bytes_equal(gpu, ref, rows=None) -> bool:
    gq, gs, gg = np_(gpu[0]), np_(gpu[1]), np_(gpu[2])
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    return bool(np.array_equal(gq, ref[0]) and np.array_equal(gs, ref[1])
                and np.float32(gg[0]).view(np.uint32) == np.float32(ref[2]).view(np.uint32))


def errors(y, y_ref, bound):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(rel.max()) if rel.size else 0.0
    return {"max_err_over_sum_abs_xw": worst, "fraction_of_tolerance": worst / 1e-5,
            "outputs_checked": int(err.size)}


def report(name, **kw):
    print(json.dumps({"workload": name, **kw}), flush=True)


def dense(config: int, cfg, rows, cols, quant_rows=None):
    t0 = time.perf_counter()
    x_cpu, w_cpu = wl.gemm_inputs(config, cfg)
    a = nv.nvfp4_quantize(x_cpu.cuda())
    b = nv.nvfp4_quantize(w_cpu.cuda())
    y = nv.nvfp4_gemm(a, b, "f32")
    torch.cuda.synchronize()
    r_idx = torch.from_numpy(rows) if rows is not None else slice(None)
    c_idx = torch.from_numpy(cols) if cols is not None else slice(None)
    ra = oracle_quantize(x_cpu[r_idx], oracle_global_scale(x_cpu))
    rb = oracle_quantize(w_cpu[c_idx], oracle_global_scale(w_cpu))
    y_ref, bound = gemm_ref(*ra, *rb)
    yn = np_(y)
    if rows is not None:
        yn = yn[rows]
    if cols is not None:
        yn = yn[:, cols]
    report(cfg.name, quantize_bytes_equal=bytes_equal(a, ra, rows) and bytes_equal(b, rb, cols),
           seeds=[wl.seed_for(config, 0), wl.seed_for(config, 1)],
           seconds=round(time.perf_counter() - t0, 1), **errors(yn, y_ref, bound))


def moe(proj: str):
    t0 = time.perf_counter()
    N, K = wl.MOE_GATE_UP if proj == "gate_up" else wl.MOE_DOWN
    routing = wl.moe_routing(wl.seed_for(3, 0))
    E, total, dev = wl.MOE_EXPERTS, int(routing.m_offsets[-1]), "cuda"
    if proj == "gate_up":
        x_cpu = wl.randn((wl.MOE_TOKENS, K), wl.seed_for(3, 1), "bf16")
        q, s, g = nv.nvfp4_quantize(x_cpu.cuda())
        a, row_index, rows_tok = (q, s, g), routing.row_token.to(dev).to(torch.int32), routing.row_token
    else:
        x_cpu = wl.randn((total, K), wl.seed_for(3, 2), "bf16")
        a, row_index, rows_tok = nv.nvfp4_quantize(x_cpu.cuda()), None, torch.arange(total)
    bq = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    bs = torch.empty((E, N, K // 16), dtype=torch.uint8, device=dev)
    bg = torch.empty((E,), dtype=torch.float32, device=dev)
    wseed = lambda e: wl.seed_for(3, (100 if proj == "gate_up" else 1000) + e)  # noqa: E731
    for e in range(E):
        nv.nvfp4_quantize(wl.randn((N, K), wseed(e), "bf16", device=dev), out=(bq[e], bs[e], bg[e:e + 1]))
    y = nv.nvfp4_grouped_gemm(routing.m_offsets.to(dev), total, a, (bq, bs, bg), "f32",
                              row_index=row_index)
    torch.cuda.synchronize()
    y_np = np_(y)
    cols = np.sort(np.random.default_rng(7).choice(N, 256, replace=False))
    off = routing.m_offsets.numpy()
    ga = oracle_global_scale(x_cpu)
    worst, checked, same = 0.0, 0, True
    for e in (0, 97, 255):
        r0, r1 = int(off[e]), int(off[e + 1])
        w_cpu = wl.randn((N, K), wseed(e), "bf16", device=dev).cpu()
        rb = oracle_quantize(w_cpu[torch.from_numpy(cols)], oracle_global_scale(w_cpu))
        same &= bytes_equal((bq[e], bs[e], bg[e:e + 1]), rb, cols)
        ra = oracle_quantize(x_cpu[rows_tok[r0:r1]], ga)
        y_ref, bound = gemm_ref(*ra, *rb)
        r = errors(y_np[r0:r1][:, cols], y_ref, bound)
        worst = max(worst, r["max_err_over_sum_abs_xw"])
        checked += r["outputs_checked"]
    report(f"moe_{proj}" + ("_through_index" if row_index is not None else ""),
           quantize_bytes_equal=same, seeds="3000-3002, 3100+e / 4000+e per expert",
           seconds=round(time.perf_counter() - t0, 1), max_err_over_sum_abs_xw=worst,
           fraction_of_tolerance=worst / 1e-5, outputs_checked=checked)


def main():
    assert torch.cuda.is_available(), "the parity report needs a GPU"
    dense(0, wl.TINY, None, None)
    rng = np.random.default_rng(11)
    dense(1, wl.LINEAR, np.sort(rng.choice(wl.LINEAR.M, 256, replace=False)),
          np.sort(rng.choice(wl.LINEAR.N, 256, replace=False)))
    for m in (1, 16, 32):
        cfg = wl.DECODE[m]
        dense(2, cfg, None, np.sort(np.random.default_rng(m).choice(cfg.N, 1024, replace=False)))
    moe("gate_up")
    moe("down")
    rng = np.random.default_rng(5)
    dense(4, wl.LARGE, np.sort(rng.choice(wl.LARGE.M, 32, replace=False)),
          np.sort(rng.choice(wl.LARGE.N, 32, replace=False)))


if __name__ == "__main__":
    main()
