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
