"""The shared tile counter of the collective kernels (snac_tuning.tile_schedule).

Long launches whose tiles each read and write many buffers take their first
grid-stride rounds as before and the remaining tiles, in order, from a
counter in the context that the last workgroup resets.  These tests check:

* every collective with the counter forced on gives the bits of the
  grid-stride schedule and of the oracle (aligned and misaligned buffers,
  several rank counts and types);
* the counter is clean for the next call: many calls in a row, more than
  the context has counter slots, of two collectives, each with its outputs
  zeroed first so that a skipped tile would show;
* graph replays of pooled calls, with eager work between the replays;
* a context re-armed by snac_check after a device-side timeout.
"""
from __future__ import annotations

import contextlib

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MiB = 1 << 20
ESIZE = {"bf16": 2, "f32": 4, "u32": 4, "byte": 1}


@contextlib.contextmanager
def schedule(v: int):
    t0 = snac.snac_get_tuning()
    snac.snac_set_tuning(tile_schedule=v)
    try:
        yield
    finally:
        snac.snac_set_tuning(**t0)


def gen(n, m, dtype, seed):
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "u32":
        return [wl.raw_u32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


# (collective, N, dtype, per-rank elements or V total, buffer offsets in elements)
CASES = [
    ("all_reduce", 8, "bf16", 12 * MiB + 1027, 0),
    ("all_reduce", 3, "f32", 5 * MiB + 17, 3),
    ("reduce_scatter", 8, "bf16", 12 * MiB, 0),
    ("reduce_scatter", 16, "f32", 4 * MiB, 1),
    ("all_gather", 8, "bf16", 4 * MiB + 5, 0),
    ("all_gather", 8, "u32", 2 * MiB + 3, 2),
    ("all_to_all", 8, "u32", 4 * MiB, 0),
    ("all_to_all", 4, "byte", 16 * MiB + 12, 5),
    ("all_gather_v", 8, "u32", 3 * MiB + 11, 0),
    ("reduce_scatter_v", 16, "f32", 6 * MiB, 0),
    ("all_to_all_v", 8, "byte", 14 * MiB, 3),
]


def run(ctx, coll, n, dtype, m, src, dst, counts):
    sp, dp, e = [b.ptr for b in src], [b.ptr for b in dst], ESIZE[dtype]
    if coll == "all_reduce":
        snac.snac_all_reduce(ctx, sp, dp, m * e, dtype)
    elif coll == "reduce_scatter":
        snac.snac_reduce_scatter(ctx, sp, dp, m * e, dtype)
    elif coll == "all_gather":
        snac.snac_all_gather(ctx, sp, dp, m * e, dtype)
    elif coll == "all_to_all":
        snac.snac_all_to_all(ctx, sp, dp, m * e, dtype)
    elif coll == "all_gather_v":
        snac.snac_all_gather_v(ctx, sp, dp, counts, dtype)
    elif coll == "reduce_scatter_v":
        snac.snac_reduce_scatter_v(ctx, sp, dp, counts, dtype)
    else:
        snac.snac_all_to_all_v(ctx, sp, dp, np.asarray(counts).reshape(-1).tolist(), dtype)


@pytest.mark.parametrize("coll,n,dtype,m,off", CASES, ids=[f"{c[0]}-n{c[1]}-{c[2]}-o{c[4]}" for c in CASES])
def test_counter_schedule_matches_grid_stride_and_oracle(coll, n, dtype, m, off):
    import torch

    e = ESIZE[dtype]
    counts = None
    if coll in ("all_gather_v", "reduce_scatter_v"):
        counts = [int(c) for c in wl.v_counts(n, m, 1, cfg=wl.CFG_TEST, seed=11)[0]]
    elif coll == "all_to_all_v":
        counts = wl.v_counts(n, m, n, cfg=wl.CFG_TEST, seed=11)
    ins = counts if coll == "all_gather_v" else [m] * n
    xs = [x[:k] for x, k in zip(gen(n, max(ins), dtype, 7), ins)]
    if coll == "all_reduce":
        want = oracle.all_reduce(xs, dtype)
    elif coll == "reduce_scatter":
        want = oracle.reduce_scatter(xs, dtype)
    elif coll == "all_gather":
        want = oracle.all_gather(xs)
    elif coll == "all_to_all":
        want = oracle.all_to_all(xs)
    elif coll == "all_gather_v":
        want = oracle.all_gather_v(xs, counts)
    elif coll == "reduce_scatter_v":
        want = oracle.reduce_scatter_v(xs, counts, dtype)
    else:
        want = oracle.all_to_all_v(xs, counts)
    src = [DevBuf(x.nbytes, offset=off * e, data=x) for x in xs]
    ctx = snac.snac_init(n, 0)
    try:
        got = {}
        for sched in (1, 2):
            dst = [DevBuf(np.asarray(w).nbytes, offset=off * e) for w in want]
            with schedule(sched):
                run(ctx, coll, n, dtype, m, src, dst, counts)
            torch.cuda.synchronize()
            snac.snac_check(ctx)
            got[sched] = [b.download(np_dtype(dtype)) for b in dst]
            for r, b in enumerate(dst):
                assert b.guards_ok(), f"schedule {sched}: canary overwritten around dst[{r}]"
        for r, w in enumerate(want):
            assert np.array_equal(got[1][r].view(np.uint8), got[2][r].view(np.uint8)), f"dst[{r}]: schedules differ"
            assert_same(got[2][r], np.asarray(w), dtype, f"{coll} N={n} {dtype} counter schedule dst[{r}]")
    finally:
        snac.snac_finalize(ctx)


@pytest.fixture(scope="module")
def big():
    """AllReduce and ReduceScatter bf16 N=8 at 64 MiB per rank (the default
    schedule uses the counter for both), with grid-stride references."""
    import torch

    n, m = 8, 32 * MiB
    ctx = snac.snac_init(n, 0)
    src = [torch.from_numpy(x.view(np.uint8)).cuda() for x in gen(n, m, "bf16", 3)]
    ar = [torch.empty(2 * m, dtype=torch.uint8, device="cuda") for _ in range(n)]
    rs = [torch.empty(2 * m // n, dtype=torch.uint8, device="cuda") for _ in range(n)]
    with schedule(1):
        snac.snac_all_reduce(ctx, src, ar, 2 * m, "bf16")
        snac.snac_reduce_scatter(ctx, src, rs, 2 * m, "bf16")
    torch.cuda.synchronize()
    ref_ar = [t.clone() for t in ar]
    ref_rs = [t.clone() for t in rs]
    # the grid-stride reference against the oracle on a slice of each output
    xs = [s[:2 * 65536].cpu().numpy().view(np.uint16) for s in src]
    assert_same(ref_ar[5][:2 * 65536].cpu().numpy().view(np.uint16), oracle.all_reduce(xs, "bf16")[5], "bf16",
                "reference AllReduce")
    yield dict(n=n, m=m, ctx=ctx, src=src, ar=ar, rs=rs, ref_ar=ref_ar, ref_rs=ref_rs)
    snac.snac_finalize(ctx)


def _equal(outs, refs):
    import torch

    return all(bool(torch.equal(a, b)) for a, b in zip(outs, refs))


def test_counter_clean_across_many_calls(big):
    import torch

    b = big
    calls = 0
    with schedule(0):
        for i in range(70):  # more calls than the context has counter slots
            outs, refs = (b["ar"], b["ref_ar"]) if i % 3 else (b["rs"], b["ref_rs"])
            for t in outs:
                t.zero_()
            if i % 3:
                snac.snac_all_reduce(b["ctx"], b["src"], outs, 2 * b["m"], "bf16")
            else:
                snac.snac_reduce_scatter(b["ctx"], b["src"], outs, 2 * b["m"], "bf16")
            calls += 1
            assert _equal(outs, refs), f"call {i}: differs from the grid-stride result"
    torch.cuda.synchronize()
    snac.snac_check(b["ctx"])
    assert calls == 70


def test_counter_in_graph_replays(big):
    import torch

    b = big
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with schedule(0):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            # warm-up outside the capture, then capture two pooled calls
            snac.snac_all_reduce(b["ctx"], b["src"], b["ar"], 2 * b["m"], "bf16", stream)
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                snac.snac_all_reduce(b["ctx"], b["src"], b["ar"], 2 * b["m"], "bf16", stream)
                snac.snac_reduce_scatter(b["ctx"], b["src"], b["rs"], 2 * b["m"], "bf16", stream)
        for rep in range(4):
            for t in b["ar"] + b["rs"]:
                t.zero_()
            # eager pooled work between replays takes other counter slots
            snac.snac_all_reduce(b["ctx"], b["src"], b["ar"], 2 * b["m"], "bf16")
            torch.cuda.synchronize()
            for t in b["ar"]:
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert _equal(b["ar"], b["ref_ar"]), f"replay {rep}: AllReduce differs"
            assert _equal(b["rs"], b["ref_rs"]), f"replay {rep}: ReduceScatter differs"
    snac.snac_check(b["ctx"])


def test_counter_after_rearm(big):
    """A device-side timeout latches, snac_check re-arms the context (every
    signal word cleared, the tile counters among them), and pooled calls
    still cover every tile."""
    import torch

    b = big
    t0 = snac.snac_get_tuning()
    try:
        snac.snac_set_tuning(spin_limit_log2=8, debug_drop_notify=2)  # rank 1 never notifies
        xs = [s[:2 * 300_000] for s in b["src"]]
        out = torch.empty(2 * 300_000, dtype=torch.uint8, device="cuda")
        snac.snac_pipeline_scale_reduce(b["ctx"], xs, out, 300_000, "bf16")
        with pytest.raises(snac.SnacError) as e:
            snac.snac_check(b["ctx"])
        assert e.value.status == snac.SNAC_E_TIMEOUT
    finally:
        snac.snac_set_tuning(**t0)
    with schedule(0):
        for t in b["ar"]:
            t.zero_()
        snac.snac_all_reduce(b["ctx"], b["src"], b["ar"], 2 * b["m"], "bf16")
        torch.cuda.synchronize()
        assert _equal(b["ar"], b["ref_ar"]), "AllReduce after re-arming differs"
    snac.snac_check(b["ctx"])
