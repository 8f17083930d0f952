"""Failure handling and graph replay on the GPU.

Failures are forced from the host so that every kernel still exits
normally: a producer's notify is suppressed by a test hook while the spin
limit of the consumers' bounded wait is tiny (timeout), or the host sets the
context's abort word before the launch (abort).  Afterwards the context must
be usable again.  Graph replay: collectives captured in a HIP graph are
replayed several times with eager work in between, each replay checked."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import assert_same, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N = 8


@pytest.fixture(scope="module")
def torch():
    import torch

    torch.cuda.set_device(0)
    return torch


@pytest.fixture
def tuning():
    t0 = snac.snac_get_tuning()
    yield snac.snac_set_tuning
    snac.snac_set_tuning(**t0)


def up(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).cuda()


def inputs(count, seed):
    return [wl.normal_bf16(count, wl.CFG_TEST, r, seed=seed) for r in range(N)]


def run_pipeline(torch, ctx, host):
    xs = [up(torch, h) for h in host]
    out = torch.empty(host[0].nbytes, dtype=torch.uint8, device="cuda")
    snac.snac_pipeline_scale_reduce(ctx, xs, out, host[0].size, "bf16")
    return out


def test_pipeline_timeout_is_reported_and_cleared(torch, tuning):
    ctx = snac.snac_init(N, 64 * 16384)
    try:
        host = inputs(300_000, 1)
        tuning(spin_limit_log2=8, debug_drop_notify=3)  # rank 2 never notifies
        run_pipeline(torch, ctx, host)
        with pytest.raises(snac.SnacError) as e:
            snac.snac_check(ctx)
        assert e.value.status == snac.SNAC_E_TIMEOUT
        tuning(spin_limit_log2=0, debug_drop_notify=0)
        out = run_pipeline(torch, ctx, host)
        snac.snac_check(ctx)
        assert_same(out.cpu().numpy().view(np.uint16), oracle.pipeline_scale_reduce(host, "bf16"), "bf16",
                    "after timeout")
    finally:
        snac.snac_finalize(ctx)


def test_pipeline_abort_is_reported_and_cleared(torch, tuning):
    ctx = snac.snac_init(N, 64 * 16384)
    try:
        host = inputs(200_000, 2)
        tuning(spin_limit_log2=30, debug_drop_notify=1)  # waits would be long: abort ends them
        snac.snac_abort(ctx)
        run_pipeline(torch, ctx, host)
        with pytest.raises(snac.SnacError) as e:
            snac.snac_check(ctx)
        assert e.value.status == snac.SNAC_E_ABORTED
        tuning(spin_limit_log2=0, debug_drop_notify=0)
        out = run_pipeline(torch, ctx, host)
        snac.snac_check(ctx)
        assert_same(out.cpu().numpy().view(np.uint16), oracle.pipeline_scale_reduce(host, "bf16"), "bf16",
                    "after abort")
    finally:
        snac.snac_finalize(ctx)


def test_finalize_reports_latched_error(torch, tuning):
    ctx = snac.snac_init(N, 64 * 16384)
    tuning(spin_limit_log2=6, debug_drop_notify=8)
    run_pipeline(torch, ctx, inputs(100_000, 3))
    with pytest.raises(snac.SnacError) as e:
        snac.snac_finalize(ctx)  # the context is freed even so
    assert e.value.status == snac.SNAC_E_TIMEOUT


def test_graph_replay(torch):
    """AllReduce, AllToAllV and the pipeline captured in one graph, replayed
    with new inputs copied in between; every replay checked."""
    ctx = snac.snac_init(N, 0)
    try:
        m = 200_003
        sets = [inputs(m, s) for s in (11, 12, 13)]
        src = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(N)]
        ar = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(N)]
        pout = torch.empty(m * 2, dtype=torch.uint8, device="cuda")
        total = 40_000
        c = wl.v_counts(N, total, N, cfg=wl.CFG_TEST)
        words = [wl.raw_u32(total, wl.CFG_TEST, r, seed=7) for r in range(N)]
        a2a_src = [up(torch, w) for w in words]
        a2a_dst = [torch.empty(int(c[:, d].sum()) * 4 + 4, dtype=torch.uint8, device="cuda") for d in range(N)]
        flat = c.reshape(-1).tolist()
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                cur = torch.cuda.current_stream()
                snac.snac_all_reduce(ctx, src, ar, m * 2, "bf16", cur)
                snac.snac_all_to_all_v(ctx, a2a_src, a2a_dst, flat, "u32", cur)
                snac.snac_pipeline_scale_reduce(ctx, src, pout, m, "bf16", cur)
        want_a2a = oracle.all_to_all_v(words, c)
        for it, host in enumerate(sets + sets[:1]):
            for t, h in zip(src, host):
                t.copy_(up(torch, h))  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            snac.snac_check(ctx)
            want = oracle.reduce_n(host, "bf16")
            for r in (0, N - 1):
                assert_same(ar[r].cpu().numpy().view(np.uint16), want, "bf16", f"replay {it} AR dst[{r}]")
            assert_same(pout.cpu().numpy().view(np.uint16), oracle.pipeline_scale_reduce(host, "bf16"), "bf16",
                        f"replay {it} pipeline")
            for d in range(N):
                got = a2a_dst[d][: want_a2a[d].nbytes].cpu().numpy().view(np.uint32)
                assert np.array_equal(got, want_a2a[d]), f"replay {it} A2AV dst[{d}]"
    finally:
        snac.snac_finalize(ctx)


def test_graph_replay_every_other_entry_point(torch):
    """ReduceScatter, AllGather, AllGatherV, ReduceScatterV, copy, reduce_n
    and the atomic AllReduce captured in one graph on a side stream, replayed
    with new inputs copied in between; every replay checked against the
    oracle.  The atomic mode gets small-integer inputs, whose sums are exact
    in any order of the adds."""
    from oracle.bf16 import f32_to_bf16

    ctx = snac.snac_init(N, 0)
    try:
        m = N * 25_001
        i = np.arange(m)
        sets = [inputs(m, s) for s in (21, 22, 23)]
        ints = [[f32_to_bf16(((k + s) * (i % 7)).astype(np.float32)) for k in range(N)] for s in (1, 2, 3)]
        src = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(N)]
        isrc = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(N)]
        rs = [torch.empty(m * 2 // N, dtype=torch.uint8, device="cuda") for _ in range(N)]
        ag = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(N)]
        c_rsv = wl.v_counts(N, m, 1, cfg=wl.CFG_TEST, seed=3)[0]
        rsv = [torch.empty(max(1, int(c)) * 2, dtype=torch.uint8, device="cuda") for c in c_rsv]
        c_agv = wl.v_counts(N, 30_000, 1, cfg=wl.CFG_TEST, seed=4)[0]
        words = [wl.raw_u32(int(c), wl.CFG_TEST, r, seed=9) for r, c in enumerate(c_agv)]
        agv_src = [up(torch, w) if w.size else torch.empty(4, dtype=torch.uint8, device="cuda") for w in words]
        agv = [torch.empty(int(c_agv.sum()) * 4, dtype=torch.uint8, device="cuda") for _ in range(N)]
        cp = torch.empty(m * 2, dtype=torch.uint8, device="cuda")
        rn = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(2)]
        at = [torch.empty(m * 2, dtype=torch.uint8, device="cuda") for _ in range(N)]
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                cur = torch.cuda.current_stream()
                snac.snac_reduce_scatter(ctx, src, rs, m * 2, "bf16", cur)
                snac.snac_all_gather(ctx, rs, ag, m * 2 // N, "bf16", cur)
                snac.snac_all_gather_v(ctx, agv_src, agv, [int(c) for c in c_agv], "u32", cur)
                snac.snac_reduce_scatter_v(ctx, src, rsv, [int(c) for c in c_rsv], "bf16", cur)
                snac.snac_copy(cp, src[0], m * 2, cur)
                snac.snac_reduce_n(rn, src[:3], m, "bf16", cur)
                snac.snac_all_reduce_ex(ctx, isrc, at, m * 2, "bf16", "atomic", cur)
        want_agv = oracle.all_gather_v(words, [int(c) for c in c_agv])
        for it, (host, ihost) in enumerate(zip(sets + sets[:1], ints + ints[:1])):
            for t, h in zip(src, host):
                t.copy_(up(torch, h))  # eager work between replays
            for t, h in zip(isrc, ihost):
                t.copy_(up(torch, h))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            snac.snac_check(ctx)
            want_rs = oracle.reduce_scatter(host, "bf16")
            want_ag = oracle.all_gather(want_rs)
            want_rsv = oracle.reduce_scatter_v(host, [int(c) for c in c_rsv], "bf16")
            want_rn = oracle.reduce_n(host[:3], "bf16")
            want_at = oracle.all_reduce(ihost, "bf16")
            for r in range(N):
                assert_same(rs[r].cpu().numpy().view(np.uint16), want_rs[r], "bf16", f"replay {it} RS dst[{r}]")
                assert_same(ag[r].cpu().numpy().view(np.uint16), want_ag[r], "bf16", f"replay {it} AG dst[{r}]")
                if c_rsv[r]:
                    got = rsv[r][: int(c_rsv[r]) * 2].cpu().numpy().view(np.uint16)
                    assert_same(got, want_rsv[r], "bf16", f"replay {it} RSV dst[{r}]")
                assert np.array_equal(agv[r].cpu().numpy().view(np.uint32), want_agv[r]), f"replay {it} AGV dst[{r}]"
                assert_same(at[r].cpu().numpy().view(np.uint16), want_at[r], "bf16", f"replay {it} atomic dst[{r}]")
            assert np.array_equal(cp.cpu().numpy(), host[0].view(np.uint8)), f"replay {it} copy"
            for k in range(2):
                assert_same(rn[k].cpu().numpy().view(np.uint16), want_rn, "bf16", f"replay {it} reduce_n dst[{k}]")
    finally:
        snac.snac_finalize(ctx)
