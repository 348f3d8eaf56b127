"""Benchmark of the NVFP4 block-scaled GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the NVFP4 linear layer M=4096, in_features K=8192, out_features
N=8192 (kernelindex "NVFP4 linear layer" shape; M is not published there),
x and W ~ N(0,1) bf16, bf16 output.  One step is the whole hot path for one
batch: quantise the activations x to NVFP4 (amax + encode kernels), then the
NVFP4 GEMM y = x . W^T.  W is quantised once ahead of time, as a layer's
weights are (leverageai "blackwell-nvfp4-gemm-optimization", "What is this?":
quantisation may happen ahead of execution).

Prints one JSON line.  ``value`` is 2*M*N*K flop per step / step time
(TFLOP/s), so the activation quantisation is charged to the step.
``roofline`` describes the GEMM kernel alone: algorithmic flop per launch
over its average launch time (HIP events on the launch stream) against the
fp16 dense matrix-core peak, since that is the MFMA family the kernel
issues.  ``decode_m16`` is the skinny M=16 GEMM over 16 rotating copies of W
(604 MB, so the 256 MB Infinity Cache cannot hold them), against HBM peak.
``cpu_baseline`` times the CPU oracle on a bounded row slice of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_linear_m4096_n8192_k8192.json")
GEMM_SOURCES = ["gemm_mfma.hip", "nvfp4_device.h"]


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_gemm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, only
    while the kernel source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash(GEMM_SOURCES):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(x_cpu, w_cpu, rows: int):
    """Time the CPU oracle on the step restricted to ``rows`` rows of x:
    quantise those rows (oracle), then the oracle GEMM against W (whose
    quantisation happens ahead of time and is not timed)."""
    import numpy as np
    from oracle import gemm_ref, global_scale_ref, quantize_ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    xs = x_cpu[:rows].float().numpy()
    gx = global_scale_ref(x_cpu.float().numpy())
    wq = quantize_ref(w_cpu.float().numpy())
    t0 = time.perf_counter()
    xq = quantize_ref(xs, global_scale=gx)
    gemm_ref(*xq, *wq)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * w_cpu.shape[0] * w_cpu.shape[1]
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{rows} of {x_cpu.shape[0]} rows of x: oracle quantise of the rows + "
                      f"oracle fp64 GEMM against the full W ({dt:.2f} s; W quantised ahead, "
                      f"untimed; {len(os.sched_getaffinity(0))} host cores visible)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["bench", "copy"], default="bench",
                    help="copy: a plain 1 GiB device copy, for HBM counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_block_scaled_gemm_amd as nv
    import workloads as wl

    dev = torch.device("cuda")
    if args.mode == "copy":
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_copy": src.numel() * 4,
                          "bytes_written_per_copy": src.numel() * 4, "copies": args.steps}))
        return

    cfg = wl.LINEAR
    M, N, K = cfg.M, cfg.N, cfg.K
    x_cpu, w_cpu = wl.gemm_inputs(1, cfg)
    x = x_cpu.to(dev)
    w = w_cpu.to(dev)
    wq = nv.nvfp4_quantize(w)                         # ahead of time
    xq = nv.nvfp4_quantize(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(nv.nvfp4_quantize_workspace_bytes(M, K), 4), dtype=torch.uint8,
                     device=dev)

    def step():
        nv.nvfp4_quantize(x, out=xq, workspace=ws)
        nv.nvfp4_gemm(xq, wq, "bf16", y=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        nv.nvfp4_quantize(x, out=xq, workspace=ws)
        ev[i][0].record(stream)
        nv.nvfp4_gemm(xq, wq, "bf16", y=y)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gemm_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    flop = 2.0 * M * N * K
    value = flop / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flop / (gemm_ms * 1e-3) / 1e12

    # skinny decode M=16 over rotating weight copies (cache-cold W)
    dcfg = wl.DECODE[16]
    xd = nv.nvfp4_quantize(wl.randn((16, dcfg.K), wl.seed_for(2, 0), "bf16").to(dev))
    copies = [tuple(t.clone() for t in wq) for _ in range(16)]
    yd = torch.empty((16, dcfg.N), dtype=torch.bfloat16, device=dev)
    for c in copies:
        nv.nvfp4_gemm(xd, c, "bf16", y=yd)
    reps = 8
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps * len(copies))]
    torch.cuda.synchronize()
    for i in range(reps * len(copies)):
        dev_ev[i][0].record(stream)
        nv.nvfp4_gemm(xd, copies[i % len(copies)], "bf16", y=yd)
        dev_ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = sum(a.elapsed_time(b) for a, b in dev_ev) / len(dev_ev)
    dec_bytes = (dcfg.N * dcfg.K * 9 // 16) + (16 * dcfg.K * 9 // 16) + 16 * dcfg.N * 2
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9

    out = {
        "metric": "NVFP4 GEMM TFLOPS + % of MFMA/HBM roofline (M=4096,N=K=8192; M=16 decode)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, fp16 MFMA products, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded N(0,1) bf16 x and W)",
        "config": {"workload": cfg.name, "M": M, "N": N, "K": K,
                   "step": "quantize x (amax+encode) + nvfp4_gemm; W quantized ahead"},
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_us": round(gemm_ms * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": measured_traffic()},
        "decode_m16": {"workload": dcfg.name, "us": round(dec_ms * 1e3, 3),
                       "algorithmic_bytes": dec_bytes, "achieved_GBps": round(dec_gbs, 1),
                       "peak_GBps": PEAK_HBM_GBS, "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                       "tflops": round(2.0 * 16 * dcfg.N * dcfg.K / (dec_ms * 1e-3) / 1e12, 3),
                       "weights": "16 rotating copies (cache-cold)"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_cpu, w_cpu, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
