"""The boundary's stream contract on the GPU: every entry point enqueues on
the stream it is given (a side stream here, never the null stream), and a
step of the path (quantise -> GEMM -> NVFP4-output GEMM -> grouped GEMM
through the routing index) can be captured into a HIP graph and replayed:
the library allocates nothing and issues no memset.  Every replay, with
eager work and synchronisations between replays, must reproduce the eager
results bit for bit (all kernels are deterministic)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from tests.gpu_util import need_gpu, note

pytestmark = pytest.mark.gpu


def _setup(seed=5):
    dev = "cuda"
    x = wl.randn((512, 1024), seed, "bf16").to(dev)
    w = wl.randn((768, 1024), seed + 1, "bf16").to(dev)
    wq = nv.nvfp4_quantize(w)
    counts = [40, 0, 70, 18, 100]
    off = wl.ragged_offsets(counts).to(dev)
    total = sum(counts)
    bq = torch.stack([wq[0][:256]] * len(counts)).contiguous()
    bs = torch.stack([wq[1][:256]] * len(counts)).contiguous()
    bg = wq[2].repeat(len(counts))
    idx = torch.from_numpy(np.random.default_rng(seed).integers(0, 512, total).astype(np.int32)).to(dev)
    bufs = dict(
        xq=(torch.empty((512, 512), dtype=torch.uint8, device=dev),
            torch.empty((512, 64), dtype=torch.uint8, device=dev),
            torch.empty(1, device=dev)),
        ws=torch.empty(max(nv.nvfp4_quantize_workspace_bytes(512, 1024), 4), dtype=torch.uint8,
                       device=dev),
        y=torch.empty((512, 768), dtype=torch.bfloat16, device=dev),
        yq=(torch.empty((512, 384), dtype=torch.uint8, device=dev),
            torch.empty((512, 48), dtype=torch.uint8, device=dev)),
        yg=torch.tensor([0.01], device=dev),
        yt=torch.empty((total, 256), dtype=torch.float32, device=dev))
    return x, wq, (off, total, (bq, bs, bg), idx), bufs


def _step(x, wq, grouped, b, stream=None):
    off, total, bw, idx = grouped
    nv.nvfp4_quantize(x, out=b["xq"], workspace=b["ws"], stream=stream)
    nv.nvfp4_gemm(b["xq"], wq, "bf16", y=b["y"], stream=stream)
    nv.nvfp4_gemm_nvfp4_out(b["xq"], wq, b["yg"], out=b["yq"], stream=stream)
    nv.nvfp4_grouped_gemm(off, total, b["xq"], bw, "f32", y=b["yt"], stream=stream,
                          row_index=idx)


def _snapshot(b):
    return [t.clone() for t in (*b["xq"], b["y"], *b["yq"], b["yt"])]


def test_side_stream():
    need_gpu()
    x, wq, grouped, b = _setup()
    _step(x, wq, grouped, b)
    torch.cuda.synchronize()
    ref = _snapshot(b)
    for t in (*b["xq"], b["y"], *b["yq"], b["yt"]):
        t.zero_()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    note("entry points on a side stream")
    with torch.cuda.stream(side):
        _step(x, wq, grouped, b, stream=side)
    side.synchronize()
    for r, g in zip(ref, _snapshot(b)):
        assert torch.equal(r, g)


def test_graph_capture_and_replay():
    need_gpu()
    x, wq, grouped, b = _setup(seed=9)
    _step(x, wq, grouped, b)          # eager (also warms up the launchers)
    torch.cuda.synchronize()
    ref = _snapshot(b)
    g = torch.cuda.CUDAGraph()
    for t in (*b["xq"], b["y"], *b["yq"], b["yt"]):
        t.zero_()
    torch.cuda.synchronize()
    note("capture the step into a graph")
    with torch.cuda.graph(g):
        _step(x, wq, grouped, b)
    for rep in range(3):
        for t in (*b["xq"], b["y"], *b["yq"], b["yt"]):
            t.fill_(3)                # eager work between replays
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for r, got in zip(ref, _snapshot(b)):
            assert torch.equal(r, got), f"replay {rep} differs"


def test_side_stream_without_context_static_scale():
    """stream=side with torch's current stream left as it is: the wrapper's
    own torch work (the static scale copied into g, freshly allocated
    outputs) must be ordered on the side stream too.  The current stream is
    kept busy meanwhile, so work left on it would land after the kernels
    that need it."""
    need_gpu()
    dev = "cuda"
    x = wl.randn((256, 1024), 21, "bf16").to(dev)
    w = wl.randn((384, 1024), 22, "bf16").to(dev)
    gs = torch.tensor([0.0029], dtype=torch.float32, device=dev)
    ref_x = nv.nvfp4_quantize(x, global_scale=gs)
    wq = nv.nvfp4_quantize(w)
    ref_y = nv.nvfp4_gemm(ref_x, wq, "f32")
    ref_o = nv.nvfp4_gemm_nvfp4_out(ref_x, wq, gs)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    note("entry points with stream=side, current stream busy")
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(100_000_000)          # ~50 ms of spinning on the current stream
    else:  # pragma: no cover
        big = torch.randn((4096, 4096), device=dev)
        for _ in range(20):
            big = big @ big.t() * 1e-3
    got_x = nv.nvfp4_quantize(x, global_scale=gs, stream=side)
    got_y = nv.nvfp4_gemm(got_x, wq, "f32", stream=side)
    got_o = nv.nvfp4_gemm_nvfp4_out(got_x, wq, gs, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    for r, g in zip(ref_x, got_x):
        assert torch.equal(r, g)
    assert torch.equal(ref_y, got_y)
    for r, g in zip(ref_o, got_o):
        assert torch.equal(r, g)


def test_graph_decode_kernels_and_grouped_multi():
    """The decode kernels (1, 4, 16 and 32 tokens at K = 8192: the
    whole-row and LDS-ring weight streams) and a two-problem grouped launch
    captured into one graph; every replay reproduces the eager results."""
    need_gpu()
    dev = "cuda"
    w = nv.nvfp4_quantize(wl.randn((1024, 8192), 21, "bf16").to(dev))
    xs = {m: nv.nvfp4_quantize(wl.randn((m, 8192), 22 + m, "bf16").to(dev)) for m in (1, 4, 16, 32)}
    ys = {m: torch.empty((m, 1024), dtype=torch.bfloat16, device=dev) for m in xs}
    counts = [5, 0, 40, 3]
    off = wl.ragged_offsets(counts).to(dev)
    total = sum(counts)
    wg = nv.nvfp4_quantize(wl.randn((4 * 256, 1024), 30, "bf16").to(dev))
    bw = (wg[0].view(4, 256, 512), wg[1].view(4, 256, 64), wg[2].repeat(4))
    a = nv.nvfp4_quantize(wl.randn((64, 1024), 31, "bf16").to(dev))
    idx = torch.from_numpy(np.random.default_rng(3).integers(0, 64, total).astype(np.int32)).to(dev)
    a2 = nv.nvfp4_quantize(wl.randn((total, 1024), 32, "bf16").to(dev))
    yg = [torch.empty((total, 256), dtype=torch.float32, device=dev) for _ in range(2)]
    calls = [dict(m_offsets=off, total_m=total, a=a, b=bw, out_dtype="f32", y=yg[0], row_index=idx),
             dict(m_offsets=off, total_m=total, a=a2, b=bw, out_dtype="f32", y=yg[1])]

    def step():
        for m in xs:
            nv.nvfp4_gemm(xs[m], w, "bf16", y=ys[m])
        nv.nvfp4_grouped_gemm_multi(calls)

    outs = [*ys.values(), *yg]
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    note("capture decode GEMMs and a grouped launch")
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(3)
        torch.cuda.synchronize()
        note(f"decode graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for r, got in zip(ref, outs):
            assert torch.equal(r, got), f"replay {rep} differs"
