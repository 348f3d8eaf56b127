"""GPU grouped (per-expert) GEMM vs the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from oracle import check_gemm, gemm_ref, global_scale_ref, grouped_gemm_ref, pack_nibbles
from tests.gpu_util import (assert_bytes_equal, need_gpu, note, np_, oracle_global_scale,
                            oracle_quantize)

pytestmark = pytest.mark.gpu


def _rand_packed(rng, shape_rows, K):
    q = rng.integers(0, 256, size=(*shape_rows, K // 2)).astype(np.uint8)
    s = rng.integers(0x10, 0x60, size=(*shape_rows, K // 16)).astype(np.uint8)
    return q, s


def _run(counts, N, K, out, seed):
    need_gpu()
    rng = np.random.default_rng(seed)
    G = len(counts)
    off = wl.ragged_offsets(counts)
    total = int(off[-1])
    aq, as_ = _rand_packed(rng, (total,), K)
    ag = np.float32(0.05)
    bq, bs = _rand_packed(rng, (G, N), K)
    bg = (rng.random(G) + 0.5).astype(np.float32)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    note(f"grouped G={G} total={total} N={N} K={K} out={out}")
    y = nv.nvfp4_grouped_gemm(off.to(dev), total, (t(aq), t(as_), torch.tensor([ag], device=dev)),
                              (t(bq), t(bs), t(bg)), out_dtype=out)
    torch.cuda.synchronize()
    y_ref, bound = grouped_gemm_ref(off.numpy(), aq, as_, ag, bq, bs, bg)
    ok, worst = check_gemm(np_(y), y_ref, bound, out)
    assert ok, worst


@pytest.mark.parametrize("counts,N,K", [
    ([3, 0, 5, 1, 0, 40], 96, 256),
    ([0, 0, 7], 64, 512),
    ([17], 48, 2048),
    ([1] * 20, 40, 256),
    ([33, 64, 2, 0, 31, 32, 130], 200, 1536),
    ([33, 0, 2, 31, 16], 72, 768),
    ([5, 9], 30, 48),
    # experts of 31 to 200 rows: chunk runs ending in 1 to 32 tokens, on a
    # ragged last weight tile
    ([63, 64, 65, 0, 96, 97, 31, 128, 129, 200, 1], 136, 1024),
])
def test_ragged_groups(counts, N, K):
    for out in ("f32", "bf16"):
        _run(counts, N, K, out, seed=sum(counts) + N + K)


@pytest.mark.parametrize("counts", [[512], [0, 512, 512], [5], [20, 0, 17, 3]])
def test_exhaustive_dequant_identity(counts):
    """Each group's A rows are one-hot rows (nibble 1.0, scale 1.0, g = 1) and
    each expert's W [8, 512] holds every nibble under every finite scale byte,
    so each group's y is exactly columns of W_e_dq, read back bit for bit.
    A group of 512 rows reads every column of its expert (all 4096
    nibble/scale pairs); the small groups run chunks with one and with two
    16-token fragments.  K = 512 runs the streaming grouped kernel."""
    need_gpu()
    K, N = 512, 8
    G = len(counts)
    off = wl.ragged_offsets(counts)
    total = int(off[-1])
    nib = np.zeros((total, K), dtype=np.uint8)
    for e in range(G):
        for i in range(int(off[e]), int(off[e + 1])):
            nib[i, 37 * (i - int(off[e])) % K] = 0x2   # 37 is odd: distinct columns
    aq = pack_nibbles(nib)
    as_ = np.full((total, K // 16), 0x38, np.uint8)
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x3F, 0xBF                 # NaN codes replaced
    rng = np.random.default_rng(1)
    bq = np.zeros((G, N, K // 2), dtype=np.uint8)
    bs = np.zeros((G, N, K // 16), dtype=np.uint8)
    for e in range(G):
        wn = np.zeros((N, K), dtype=np.uint8)
        for blk in range(N * K // 16):
            r, c = divmod(blk, K // 16)
            wn[r, 16 * c:16 * c + 16] = rng.permutation(16)
        bq[e] = pack_nibbles(wn)
        bs[e] = np.roll(codes, 64 * e).reshape(N, K // 16)
    bg = np.ones(G, dtype=np.float32)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    note(f"grouped exhaustive dequant counts={counts}")
    y = nv.nvfp4_grouped_gemm(off.to(dev), total, (t(aq), t(as_), torch.ones(1, device=dev)),
                              (t(bq), t(bs), t(bg)), out_dtype="f32")
    torch.cuda.synchronize()
    y_ref, _ = grouped_gemm_ref(off.numpy(), aq, as_, np.float32(1), bq, bs, bg)
    assert np.array_equal(np_(y), y_ref.astype(np.float32))


@pytest.mark.parametrize("counts,N,K,a_rows", [
    ([3, 0, 5, 1, 0, 40], 96, 512, 50),
    ([33, 64, 2, 0, 31], 130, 1024, 20),
    ([7, 9], 40, 768, 12),
    ([5, 9], 30, 48, 6),
    ([63, 64, 65, 97, 129, 200], 136, 1024, 300),
])
def test_gather_rows(counts, N, K, a_rows):
    """Grouped rows read through an index list (duplicates, and two indices
    outside [0, a_rows) that must read as zero rows) against the oracle on
    rows gathered on the CPU."""
    need_gpu()
    rng = np.random.default_rng(sum(counts) + N + K)
    G = len(counts)
    off = wl.ragged_offsets(counts)
    total = int(off[-1])
    aq, as_ = _rand_packed(rng, (a_rows,), K)
    idx = rng.integers(0, a_rows, size=total).astype(np.int32)
    idx[0], idx[-1] = -1, a_rows + 3
    ag = np.float32(0.05)
    bq, bs = _rand_packed(rng, (G, N), K)
    bg = (rng.random(G) + 0.5).astype(np.float32)
    valid = (idx >= 0) & (idx < a_rows)
    gq = np.where(valid[:, None], aq[np.clip(idx, 0, a_rows - 1)], 0).astype(np.uint8)
    gs = np.where(valid[:, None], as_[np.clip(idx, 0, a_rows - 1)], 0).astype(np.uint8)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    y_ref, bound = grouped_gemm_ref(off.numpy(), gq, gs, ag, bq, bs, bg)
    for out in ("f32", "bf16"):
        note(f"grouped gather G={G} total={total} a_rows={a_rows} N={N} K={K} out={out}")
        y = nv.nvfp4_grouped_gemm(off.to(dev), total, (t(aq), t(as_), torch.tensor([ag], device=dev)),
                                  (t(bq), t(bs), t(bg)), out_dtype=out, row_index=t(idx))
        torch.cuda.synchronize()
        ok, worst = check_gemm(np_(y), y_ref, bound, out)
        assert ok, (out, worst)


def test_all_groups_empty_but_last():
    _run([0] * 15 + [4], 64, 512, "f32", seed=3)


def _moe_case(proj: str, gather: bool = False):
    """MoE workload, one projection: 512 tokens routed top-8 over 256 experts
    (gate_up either on gathered token rows or through the routing index)."""
    need_gpu()
    N, K = wl.MOE_GATE_UP if proj == "gate_up" else wl.MOE_DOWN
    routing = wl.moe_routing(wl.seed_for(3, 0))
    E = wl.MOE_EXPERTS
    total = int(routing.m_offsets[-1])
    dev = "cuda"
    if proj == "gate_up":
        x_cpu = wl.randn((wl.MOE_TOKENS, K), wl.seed_for(3, 1), "bf16")
        q, s, g = nv.nvfp4_quantize(x_cpu.cuda())
        rt = routing.row_token.to(dev)
        if gather:
            a, row_index = (q, s, g), rt.to(torch.int32)
        else:
            a, row_index = (q.index_select(0, rt), s.index_select(0, rt), g), None
        rows_tok = routing.row_token
    else:
        x_cpu = wl.randn((total, K), wl.seed_for(3, 2), "bf16")
        a = nv.nvfp4_quantize(x_cpu.cuda())
        rows_tok = torch.arange(total)
        row_index = None
    bq = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    bs = torch.empty((E, N, K // 16), dtype=torch.uint8, device=dev)
    bg = torch.empty((E,), dtype=torch.float32, device=dev)
    wseed = lambda e: wl.seed_for(3, (100 if proj == "gate_up" else 1000) + e)  # noqa: E731
    note(f"moe {proj}: quantizing {E} experts")
    for e in range(E):
        w = wl.randn((N, K), wseed(e), "bf16", device=dev)
        nv.nvfp4_quantize(w, out=(bq[e], bs[e], bg[e:e + 1]))
    note(f"moe {proj}: grouped gemm")
    y = nv.nvfp4_grouped_gemm(routing.m_offsets.to(dev), total, a, (bq, bs, bg), "bf16",
                              row_index=row_index)
    torch.cuda.synchronize()
    y_np = np_(y)
    note(f"moe {proj}: oracle quantise of the activations")
    ra_all = oracle_quantize(x_cpu)
    assert_bytes_equal(q if proj == "gate_up" else a[0], s if proj == "gate_up" else a[1],
                       g if proj == "gate_up" else a[2], *ra_all)
    off = routing.m_offsets.numpy()
    rng = np.random.default_rng(7)
    note(f"moe {proj}: every expert with rows, 64 sampled output columns each")
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        cols = np.sort(rng.choice(N, 64, replace=False))
        w = wl.randn((N, K), wseed(e), "bf16", device=dev)
        # the expert's amax is an exact, order-free reduction (taken on the
        # device); the oracle turns it into the global scale
        gw = global_scale_ref(np.array([w.abs().max().float().item()], np.float32))
        w_cols = w.index_select(0, torch.from_numpy(cols).to(dev)).cpu()
        rb = oracle_quantize(w_cols, gw)
        assert_bytes_equal(bq[e], bs[e], bg[e:e + 1], *rb, rows=cols)
        rows = rows_tok[r0:r1].numpy()
        y_ref, bound = gemm_ref(ra_all[0][rows], ra_all[1][rows], ra_all[2], *rb)
        ok, worst = check_gemm(y_np[r0:r1][:, cols], y_ref, bound, "bf16")
        assert ok, (e, worst)


def test_moe_gate_up():
    _moe_case("gate_up")


def test_moe_gate_up_gather():
    _moe_case("gate_up", gather=True)


def test_moe_down():
    _moe_case("down")


@pytest.mark.parametrize("out,pad,shift", [("bf16", 4, 0), ("bf16", 1, 0), ("bf16", 4, 2),
                                           ("f32", 8, 0), ("f32", 4, 1)])
def test_strided_output(out, pad, shift):
    """y inside a wider buffer (row stride N + pad, start shifted by `shift`
    elements): aligned rows take the four-column stores, the others the
    per-element writer; the padding keeps its sentinel."""
    need_gpu()
    counts, N, K = [33, 0, 2, 31, 16, 40], 200, 512
    rng = np.random.default_rng(pad * 10 + shift)
    G = len(counts)
    off = wl.ragged_offsets(counts)
    total = int(off[-1])
    aq, as_ = _rand_packed(rng, (total,), K)
    ag = np.float32(0.05)
    bq, bs = _rand_packed(rng, (G, N), K)
    bg = (rng.random(G) + 0.5).astype(np.float32)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    ld = N + pad
    buf = torch.full((total * ld + shift + pad,), -7.0, dtype=dt, device=dev)
    y = buf[shift:shift + total * ld].view(total, ld)[:, :N]
    note(f"grouped strided output out={out} ld_y={ld} shift={shift}")
    nv.nvfp4_grouped_gemm(off.to(dev), total, (t(aq), t(as_), torch.tensor([ag], device=dev)),
                          (t(bq), t(bs), t(bg)), out_dtype=out, y=y)
    torch.cuda.synchronize()
    y_ref, bound = grouped_gemm_ref(off.numpy(), aq, as_, ag, bq, bs, bg)
    ok, worst = check_gemm(np_(y.contiguous()), y_ref, bound, out)
    assert ok, worst
    full = buf.float().cpu().numpy()
    mask = np.ones(full.shape, bool)
    mask[(shift + np.arange(total)[:, None] * ld + np.arange(N)[None, :]).ravel()] = False
    assert np.all(full[mask] == -7.0), "writes outside the output view"


@pytest.mark.parametrize("K,N", [(1024, 192), (768, 72)])
def test_skewed_routing(K, N):
    """Skewed router (a few experts take most tokens, most take none):
    experts with hundreds of rows run many 32-token chunks, the others are
    skipped; tokens are read through the routing index."""
    need_gpu()
    r = wl.moe_routing(wl.seed_for(3, 5), tokens=512, experts=64, topk=8, skew=2.0)
    counts = torch.diff(r.m_offsets.to(torch.int64))
    assert int(counts.max()) > 200 and int((counts == 0).sum()) > 10
    rng = np.random.default_rng(K + N)
    G, total = 64, int(r.m_offsets[-1])
    aq, as_ = _rand_packed(rng, (512,), K)
    ag = np.float32(0.05)
    bq, bs = _rand_packed(rng, (G, N), K)
    bg = (rng.random(G) + 0.5).astype(np.float32)
    rt = r.row_token.numpy().astype(np.int64)
    y_ref, bound = grouped_gemm_ref(r.m_offsets.numpy(), aq[rt], as_[rt], ag, bq, bs, bg)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    note(f"grouped skewed routing K={K} N={N} max_rows={int(counts.max())}")
    y = nv.nvfp4_grouped_gemm(r.m_offsets.to(dev), total,
                              (t(aq), t(as_), torch.tensor([ag], device=dev)),
                              (t(bq), t(bs), t(bg)), out_dtype="bf16",
                              row_index=r.row_token.to(torch.int32).to(dev))
    torch.cuda.synchronize()
    ok, worst = check_gemm(np_(y), y_ref, bound, "bf16")
    assert ok, worst


def test_general_kernel_past_its_row_chunks():
    """The general kernel launches at most 1,048,560 rows (65535 row tiles of
    16) at a time; larger problems run in row chunks that see global rows.
    K = 256 sends grouped calls to it.  1,100,000 grouped rows in 4 groups
    (one empty, one straddling the first chunk boundary), rows repeating a
    seeded 1000-row block; then the same through a routing index with
    repeated and out-of-range entries.  Rows at the chunk and group
    boundaries, the last rows and a random sample are checked."""
    need_gpu()
    total, K, N, period = 1_100_000, 256, 16, 1000
    bounds = [0, 500_000, 500_000, 1_048_570, total]
    ra = oracle_quantize(wl.randn((period, K), 8201, "bf16"))
    rbs = [oracle_quantize(wl.randn((N, K), 8202 + e, "bf16")) for e in range(4)]
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    off = torch.tensor(bounds, dtype=torch.int32, device=dev)
    b = (t(np.stack([r[0] for r in rbs])), t(np.stack([r[1] for r in rbs])),
         t(np.array([r[2] for r in rbs], dtype=np.float32)))
    a_g = torch.tensor([float(ra[2])], device=dev)
    reps = total // period
    a_full = (t(ra[0]).repeat(reps, 1), t(ra[1]).repeat(reps, 1), a_g)
    rng = np.random.default_rng(8210)
    rows = np.unique(np.concatenate([[0, 499_999, 500_000, 1_048_559, 1_048_560, 1_048_561,
                                      1_048_569, 1_048_570, total - 1],
                                     rng.choice(total, 8, replace=False)]))
    group = np.searchsorted(np.array(bounds), rows, side="right") - 1

    def check(y, src_rows):
        y_np = np_(y[torch.from_numpy(rows).to(dev)])
        for e in range(4):
            sel = group == e
            if not sel.any():
                continue
            src = src_rows[sel]
            ok_rows = (src >= 0) & (src < period)
            qa = np.where(ok_rows[:, None], ra[0][np.clip(src, 0, period - 1)], 0).astype(np.uint8)
            sa = np.where(ok_rows[:, None], ra[1][np.clip(src, 0, period - 1)], 0).astype(np.uint8)
            y_ref, bound = gemm_ref(qa, sa, ra[2], *rbs[e])
            ok, worst = check_gemm(y_np[sel], y_ref, bound, "f32")
            assert ok, f"group {e}: worst |err|/tol = {worst}"

    note(f"grouped general kernel total={total} K={K} N={N}")
    y = nv.nvfp4_grouped_gemm(off, total, a_full, b, out_dtype="f32")
    torch.cuda.synchronize()
    check(y, rows % period)
    del y, a_full

    idx = (np.arange(total, dtype=np.int64) * 7919) % period
    idx[[1_048_560, total - 1]] = [-1, period]               # read as zero rows
    note(f"grouped general kernel through the index total={total} a_rows={period}")
    y = nv.nvfp4_grouped_gemm(off, total, (t(ra[0]), t(ra[1]), a_g), b, out_dtype="f32",
                              row_index=t(idx.astype(np.int32)))
    torch.cuda.synchronize()
    check(y, idx[rows])


def test_more_experts_than_one_launch_piece():
    """2500 experts (one launch handles at most 1023 per problem, so the
    call runs pieces of consecutive experts), most with 0-3 rows and one
    with 70, through the streaming kernel (K = 512)."""
    rng = np.random.default_rng(2500)
    counts = (rng.integers(0, 4, size=2500) * (rng.random(2500) < 0.6)).tolist()
    counts[1700] = 70
    _run(counts, 64, 512, "f32", seed=2500)


@pytest.mark.parametrize("K", [512, 48])
def test_inconsistent_offsets_stay_inside_the_output(K):
    """Offsets that decrease and overlap (a violated precondition): the
    result is unspecified, but nothing outside y's rows [0, total_m) may be
    written and the call must finish.  K = 512 runs the streaming kernel,
    K = 48 the general one."""
    need_gpu()
    rng = np.random.default_rng(K)
    N, total = 72, 60
    off = torch.tensor([0, 50, 10, 70, -5, 60], dtype=torch.int32)
    G = len(off) - 1
    aq, as_ = _rand_packed(rng, (total,), K)
    bq, bs = _rand_packed(rng, (G, N), K)
    dev = "cuda"
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)  # noqa: E731
    buf = torch.full((total + 8, N), -7.0, dtype=torch.float32, device=dev)
    y = buf[4:4 + total]
    note(f"grouped inconsistent offsets K={K}")
    nv.nvfp4_grouped_gemm(off.to(dev), total, (t(aq), t(as_), torch.ones(1, device=dev)),
                          (t(bq), t(bs), torch.ones(G, device=dev)), out_dtype="f32", y=y)
    torch.cuda.synchronize()
    full = buf.cpu().numpy()
    assert np.all(full[:4] == -7.0) and np.all(full[4 + total:] == -7.0)
