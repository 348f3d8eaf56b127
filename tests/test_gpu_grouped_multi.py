"""Several grouped GEMMs in one launch (nvfp4_grouped_gemm_multi) vs the
oracle and vs the same problems run by separate calls, through the C ABI.

The separate calls run the same kernel on the same items with the same
per-job arithmetic, so the outputs must match them bit for bit; the oracle
check bounds both against the exact products."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_gemm_amd as nv
import workloads as wl
from oracle import check_gemm, gemm_ref, grouped_gemm_ref
from tests.gpu_util import need_gpu, note, np_

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _t(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(DEV)


def _rand_packed(rng, shape_rows, K):
    q = rng.integers(0, 256, size=(*shape_rows, K // 2)).astype(np.uint8)
    s = rng.integers(0x10, 0x60, size=(*shape_rows, K // 16)).astype(np.uint8)
    return q, s


def _problem(rng, counts, N, K, out, a_rows=None):
    """One grouped problem with host copies for the oracle.  a_rows: read
    the grouped rows through a routing index into a_rows activation rows
    (two entries out of range: zero rows)."""
    G = len(counts)
    off = wl.ragged_offsets(counts)
    total = int(off[-1])
    rows = total if a_rows is None else a_rows
    aq, as_ = _rand_packed(rng, (rows,), K)
    ag = np.float32(0.05)
    bq, bs = _rand_packed(rng, (G, N), K)
    bg = (rng.random(G) + 0.5).astype(np.float32)
    call = dict(m_offsets=off.to(DEV), total_m=total,
                a=(_t(aq), _t(as_), torch.tensor([ag], device=DEV)),
                b=(_t(bq), _t(bs), _t(bg)), out_dtype=out)
    if a_rows is None:
        gq, gs = aq, as_
    else:
        idx = rng.integers(0, a_rows, size=total).astype(np.int32)
        if total >= 2:
            idx[0], idx[-1] = -1, a_rows + 3
        ok = (idx >= 0) & (idx < a_rows)
        gq = np.where(ok[:, None], aq[np.clip(idx, 0, a_rows - 1)], 0).astype(np.uint8)
        gs = np.where(ok[:, None], as_[np.clip(idx, 0, a_rows - 1)], 0).astype(np.uint8)
        call["row_index"] = _t(idx)
    ref = (off.numpy(), gq, gs, ag, bq, bs, bg)
    return call, ref


def _separate(calls):
    return [nv.nvfp4_grouped_gemm(**c) for c in calls]


def _check(calls, refs, what):
    note(f"grouped multi {what}: one launch")
    ys = nv.nvfp4_grouped_gemm_multi(calls)
    torch.cuda.synchronize()
    note(f"grouped multi {what}: separate calls")
    ys_sep = _separate(calls)
    torch.cuda.synchronize()
    for i, (y, y_sep, ref, c) in enumerate(zip(ys, ys_sep, refs, calls)):
        assert torch.equal(y.view(torch.uint8), y_sep.view(torch.uint8)), \
            f"problem {i}: differs from its own call"
        y_ref, bound = grouped_gemm_ref(*ref)
        ok, worst = check_gemm(np_(y), y_ref, bound, c["out_dtype"])
        assert ok, (i, worst)


@pytest.mark.parametrize("specs", [
    # (counts, N, K, out, a_rows or None)
    [([3, 0, 5, 1, 0, 40], 96, 512, "bf16", 50), ([3, 0, 5, 1, 0, 40], 64, 1024, "bf16", None)],
    [([33, 64, 2, 0, 31], 130, 1536, "f32", 20), ([33, 64, 2, 0, 31], 200, 512, "f32", None)],
    [([17], 48, 2048, "bf16", None), ([0, 0, 7], 64, 512, "f32", None),
     ([1] * 20, 40, 512, "bf16", 9)],
    [([5, 9, 33, 2], 72, 1024, "f32", None)] * 4,
    [([0, 0, 0], 64, 512, "bf16", None), ([7, 1], 30, 512, "bf16", None)],
    [([63, 64, 65, 0, 129], 136, 1024, "bf16", 300), ([5, 9, 33, 2], 72, 1024, "f32", None),
     ([200, 3], 64, 512, "f32", None)],
])
def test_problems_in_one_launch(specs):
    """Ragged groups (empty experts, chunks of one and two token fragments,
    experts of up to 200 rows, ragged weight tiles),
    mixed K, N and output types, with and without a routing index, up to the
    four-problem limit."""
    need_gpu()
    rng = np.random.default_rng(sum(len(s[0]) + s[1] + s[2] for s in specs))
    pairs = [_problem(rng, *s) for s in specs]
    _check([p[0] for p in pairs], [p[1] for p in pairs], f"{len(specs)} problems")


def test_fallback_runs_each_problem():
    """K = 48 cannot stream (K % 512): the call runs each problem through its
    own dispatch, same results."""
    need_gpu()
    rng = np.random.default_rng(48)
    pairs = [_problem(rng, [5, 9], 30, 48, "f32"), _problem(rng, [3, 0, 8], 64, 512, "bf16", 12)]
    _check([p[0] for p in pairs], [p[1] for p in pairs], "fallback")


def test_skewed_pair():
    """Skewed router (a few experts hold hundreds of rows, most none):
    gate_up-like problem through the routing index and down-like problem on
    grouped rows, in one launch."""
    need_gpu()
    r = wl.moe_routing(wl.seed_for(3, 5), tokens=512, experts=64, topk=8, skew=2.0)
    counts = torch.diff(r.m_offsets.to(torch.int64)).tolist()
    assert max(counts) > 200 and sum(c == 0 for c in counts) > 10
    rng = np.random.default_rng(77)
    pairs = [_problem(rng, counts, 192, 1024, "bf16", 512), _problem(rng, counts, 128, 512, "bf16")]
    _check([p[0] for p in pairs], [p[1] for p in pairs], "skewed")


@pytest.mark.parametrize("skew", [0.0, 1.0])
def test_moe_layer_both_projections(skew):
    """The MoE workload (512 tokens, top-8 of 256 experts; gate_up N = 4096,
    K = 6144 read through the routing index; down N = 6144, K = 2048 on the
    grouped rows) in one launch: bit-equal to the two separate calls on every
    output, and a sampled expert set checked against the oracle."""
    need_gpu()
    routing = wl.moe_routing(wl.seed_for(3, 0), skew=skew)
    E, T = wl.MOE_EXPERTS, wl.MOE_TOKENS
    total = int(routing.m_offsets[-1])
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)

    def packed(rows_shape, K):
        q = torch.randint(0, 256, (*rows_shape, K // 2), dtype=torch.uint8, device=DEV, generator=g)
        s = torch.randint(0x10, 0x60, (*rows_shape, K // 16), dtype=torch.uint8, device=DEV,
                          generator=g)
        return q, s

    (Ng, Kg), (Nd, Kd) = wl.MOE_GATE_UP, wl.MOE_DOWN
    xq, xs = packed((T,), Kg)
    hq, hs = packed((total,), Kd)
    wgq, wgs = packed((E, Ng), Kg)
    wdq, wds = packed((E, Nd), Kd)
    ag = torch.tensor([0.03], device=DEV)
    bgg = torch.rand(E, device=DEV, generator=g) + 0.5
    bgd = torch.rand(E, device=DEV, generator=g) + 0.5
    off = routing.m_offsets.to(DEV)
    rt = routing.row_token.to(torch.int32).to(DEV)
    calls = [dict(m_offsets=off, total_m=total, a=(xq, xs, ag), b=(wgq, wgs, bgg),
                  out_dtype="bf16", row_index=rt),
             dict(m_offsets=off, total_m=total, a=(hq, hs, ag), b=(wdq, wds, bgd),
                  out_dtype="bf16")]
    note(f"moe both projections skew={skew}: one launch")
    y_g, y_d = nv.nvfp4_grouped_gemm_multi(calls)
    torch.cuda.synchronize()
    note(f"moe both projections skew={skew}: separate calls")
    s_g, s_d = _separate(calls)
    torch.cuda.synchronize()
    assert torch.equal(y_g.view(torch.int16), s_g.view(torch.int16))
    assert torch.equal(y_d.view(torch.int16), s_d.view(torch.int16))

    offs = routing.m_offsets.numpy()
    with_rows = [e for e in range(E) if offs[e + 1] > offs[e]]
    rng = np.random.default_rng(int(skew * 10) + 5)
    experts = sorted(set([with_rows[0], with_rows[-1]]
                         + list(rng.choice(with_rows, 6, replace=False))))
    note(f"moe both projections skew={skew}: oracle on experts {experts}")
    rtn = routing.row_token.numpy()
    yg, yd = np_(y_g), np_(y_d)
    for e in experts:
        r0, r1 = int(offs[e]), int(offs[e + 1])
        cols = np.sort(rng.choice(Ng, 48, replace=False))
        ci = torch.from_numpy(cols).to(DEV)
        rows = torch.from_numpy(rtn[r0:r1].astype(np.int64)).to(DEV)
        y_ref, bound = gemm_ref(np_(xq.index_select(0, rows)), np_(xs.index_select(0, rows)),
                                np.float32(0.03), np_(wgq[e].index_select(0, ci)),
                                np_(wgs[e].index_select(0, ci)), np.float32(bgg[e].item()))
        ok, worst = check_gemm(yg[r0:r1][:, cols], y_ref, bound, "bf16")
        assert ok, ("gate_up", e, worst)
        cols = np.sort(rng.choice(Nd, 48, replace=False))
        ci = torch.from_numpy(cols).to(DEV)
        y_ref, bound = gemm_ref(np_(hq[r0:r1]), np_(hs[r0:r1]), np.float32(0.03),
                                np_(wdq[e].index_select(0, ci)), np_(wds[e].index_select(0, ci)),
                                np.float32(bgd[e].item()))
        ok, worst = check_gemm(yd[r0:r1][:, cols], y_ref, bound, "bf16")
        assert ok, ("down", e, worst)
