"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (library defaults, one context on torch's current stream).

Every output of every configured workload is compared whole, element by
element, with the oracle (bit for bit): the AllReduce at every power of two
from 1 KiB to 1 GiB per rank, ReduceScatter then AllGather at 32768 x 2048
per rank, AllToAll, AllToAllV, AllGatherV and ReduceScatterV at 128 MiB per
rank, and the SNAC pipeline at 4096 x 8192 per rank.  Outputs of 512 MiB and
more are downloaded and compared in slices; every destination of a
replicated output is compared with destination 0 on the GPU and destination
0 with the oracle.  Bytes past each output (canaries) must be untouched.

The oracle runs on the host over slices of the inputs, several slices at a
time in threads: its functions are elementwise (reduce_n) or pure data
movement, so a slice of the output is the oracle of the same slice of the
inputs.  Host memory at the largest case: 8 GiB of inputs plus 1 GiB of
expected output.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import CANARY, assert_same, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KiB = 1 << 10
MiB = 1 << 20
GiB = 1 << 30
N = 8
GUARD = 256
SLICE = 64 * MiB  # bytes per download / compare slice
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def note(msg: str) -> None:
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch

    torch.cuda.set_device(0)
    return torch


@pytest.fixture(scope="module")
def ctx(torch):
    c = snac.snac_init(N, 0, torch.cuda.current_stream())
    yield c
    snac.snac_finalize(c, torch.cuda.current_stream())


def stream(torch):
    return torch.cuda.current_stream()


def up(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).cuda()


class Out:
    """A device output of `nbytes` with GUARD canary bytes on both sides;
    `.t` is the output itself (a view, 256-byte aligned)."""

    def __init__(self, torch, nbytes: int):
        self.nbytes = nbytes
        self.full = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.full[GUARD:GUARD + nbytes]

    def guards_ok(self) -> bool:
        lo = self.full[:GUARD]
        hi = self.full[GUARD + self.nbytes:]
        return bool((lo == CANARY).all().item()) and bool((hi == CANARY).all().item())


def compare_whole(t, want: np.ndarray, dtype: str, what: str) -> None:
    """Device byte tensor `t` against the host array `want`, whole, in
    slices of SLICE bytes; bit patterns for "u32" (a NaN matches a NaN only
    for the floating-point types, as assert_same defines)."""
    npd = {"bf16": np.uint16, "f32": np.float32, "u32": np.uint32}[dtype]
    w = np.ascontiguousarray(want).view(npd).reshape(-1)
    wb = w.view(np.uint8)
    assert t.numel() == wb.size, (what, t.numel(), wb.size)
    es = w.itemsize
    for lo in range(0, wb.size, SLICE):
        hi = min(wb.size, lo + SLICE)
        got = t[lo:hi].cpu().numpy().view(npd)
        assert_same(got, w[lo // es:hi // es], dtype, f"{what} bytes [{lo}, {hi})")


def reduce_in_slices(host: list[np.ndarray], dtype: str, lo: int = 0, hi: int | None = None,
                     slice_elems: int = 8 * MiB) -> np.ndarray:
    """oracle.reduce_n over elements [lo, hi) of every input, computed over
    slices of the element range on THREADS threads (NumPy releases the GIL in
    its loops)."""
    hi = len(host[0]) if hi is None else hi
    out = np.empty(hi - lo, dtype=host[0].dtype)
    bounds = [(a, min(hi, a + slice_elems)) for a in range(lo, hi, slice_elems)]

    def work(b):
        a, z = b
        out[a - lo:z - lo] = oracle.reduce_n([h[a:z] for h in host], dtype)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, bounds))
    return out


# ------------------------------------------------ AllReduce bf16, N = 8
def test_allreduce_bf16_n8_every_power_of_two(torch, ctx):
    """Every per-rank size 2^10 .. 2^30 bytes, each output compared whole:
    destination 0 with the oracle, destinations 1..7 with destination 0 on the
    GPU, and the 256 bytes past the output untouched.  Outputs are reset to
    the canary before each size, so a size cannot pass on what a smaller one
    wrote.  The 256 MiB headline is run twice and must repeat bit for bit."""
    top = GiB
    m = top // 2
    t0 = time.time()
    host = [wl.normal_bf16(m, wl.CFG_AR_BF16_N8, r) for r in range(N)]
    note(f"AR inputs 8 x 1 GiB in {time.time() - t0:.1f}s")
    t0 = time.time()
    want = reduce_in_slices(host, "bf16")
    note(f"AR oracle over 8 x 1 GiB in {time.time() - t0:.1f}s on {THREADS} threads")
    src = [up(torch, h) for h in host]
    del host
    dst = [torch.empty(top, dtype=torch.uint8, device="cuda") for _ in range(N)]
    st = stream(torch)
    for p in range(10, 31):
        b = 1 << p
        end = min(top, b + GUARD)
        for d in dst:
            d[:end].fill_(CANARY)
        snac.snac_all_reduce(ctx, src, dst, b, "bf16", st)
        torch.cuda.synchronize()
        for r in range(1, N):
            assert torch.equal(dst[r][:b], dst[0][:b]), f"AR {b} B/rank: dst[{r}] != dst[0]"
        if b < top:
            for r in range(N):
                assert bool((dst[r][b:end] == CANARY).all().item()), f"AR {b} B/rank wrote past dst[{r}]"
        compare_whole(dst[0][:b], want[:b // 2], "bf16", f"AR {b} B/rank dst[0]")
        if b == 256 * MiB:
            first = dst[0][:b].clone()
            snac.snac_all_reduce(ctx, src, dst, b, "bf16", st)
            torch.cuda.synchronize()
            assert torch.equal(first, dst[0][:b]), "AR 256 MiB/rank: repeat run differs"
            del first
    note("AR sweep 1 KiB .. 1 GiB per rank: every output equal to the oracle")


# ------------------------------------- ReduceScatter then AllGather, N = 8
def test_rs_then_ag_equals_allreduce(torch, ctx):
    """Config 3 whole: RS outputs against oracle.reduce_scatter, the AllGather
    of them against oracle.all_gather of the oracle's RS, the AllReduce of the
    same inputs against oracle.all_reduce, and AG(RS(x)) == AR(x) on the GPU."""
    rows, cols = N * 4096, 2048
    m = rows * cols
    per_rank = m * 2
    host = [wl.normal_bf16(m, wl.CFG_RS_AG_BF16_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    rs = [Out(torch, per_rank // N) for _ in range(N)]
    ag = [Out(torch, per_rank) for _ in range(N)]
    ar = [Out(torch, per_rank) for _ in range(N)]
    st = stream(torch)
    snac.snac_reduce_scatter(ctx, src, [o.t for o in rs], per_rank, "bf16", st)
    snac.snac_all_gather(ctx, [o.t for o in rs], [o.t for o in ag], per_rank // N, "bf16", st)
    snac.snac_all_reduce(ctx, src, [o.t for o in ar], per_rank, "bf16", st)
    torch.cuda.synchronize()
    for r in range(N):
        assert torch.equal(ag[r].t, ar[r].t), f"AG(RS(x))[{r}] != AR(x)[{r}]"
    want_rs = oracle.reduce_scatter(host, "bf16")
    for r in range(N):
        compare_whole(rs[r].t, want_rs[r], "bf16", f"RS dst[{r}]")
    want_ag = oracle.all_gather(want_rs)
    for r in range(N):
        compare_whole(ag[r].t, want_ag[r], "bf16", f"AG(RS) dst[{r}]")
    want_ar = reduce_in_slices(host, "bf16")
    compare_whole(ar[0].t, want_ar, "bf16", "AR dst[0]")
    for o in rs + ag + ar:
        assert o.guards_ok(), "a canary next to an output changed"


# ----------------------------------- AllToAll(V), AllGatherV, ReduceScatterV
@pytest.mark.parametrize("dtype", ["u32", "f32"])
def test_all_to_all_128mib(torch, ctx, dtype):
    e = 128 * MiB // 4
    host = [wl.raw_u32(e, wl.CFG_A2A_N8, r) if dtype == "u32" else wl.uniform_f32(e, wl.CFG_A2A_N8, r)
            for r in range(N)]
    src = [up(torch, h) for h in host]
    dst = [Out(torch, e * 4) for _ in range(N)]
    snac.snac_all_to_all(ctx, src, [o.t for o in dst], e * 4, dtype, stream(torch))
    torch.cuda.synchronize()
    want = oracle.all_to_all(host)
    for d in range(N):
        compare_whole(dst[d].t, want[d], "u32", f"A2A {dtype} dst[{d}]")
        assert dst[d].guards_ok(), f"A2A dst[{d}] canary"


def test_all_to_all_v_128mib(torch, ctx):
    e = 128 * MiB // 4
    c = wl.v_counts(N, e, N, cfg=wl.CFG_A2A_N8)
    assert (c == 0).any() and (c % 4 != 0).any()
    host = [wl.raw_u32(e, wl.CFG_A2A_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    want = oracle.all_to_all_v(host, c)
    dst = [Out(torch, w.nbytes) for w in want]
    snac.snac_all_to_all_v(ctx, src, [o.t for o in dst], c.reshape(-1).tolist(), "u32", stream(torch))
    torch.cuda.synchronize()
    for d in range(N):
        compare_whole(dst[d].t, want[d], "u32", f"A2AV dst[{d}]")
        assert dst[d].guards_ok(), f"A2AV dst[{d}] canary"


def test_all_gather_v_128mib(torch, ctx):
    e = 128 * MiB // 4
    c = wl.v_counts(N, e, 1, cfg=wl.CFG_A2A_N8)[0]
    assert (c == 0).any() and (c % 4 != 0).any()
    host = [wl.raw_u32(int(c[k]), wl.CFG_A2A_N8, k) for k in range(N)]
    src = [up(torch, h) if h.size else 0 for h in host]
    dst = [Out(torch, e * 4) for _ in range(N)]
    snac.snac_all_gather_v(ctx, src, [o.t for o in dst], c.tolist(), "u32", stream(torch))
    torch.cuda.synchronize()
    want = oracle.all_gather_v(host, c.tolist())
    for d in range(N):
        compare_whole(dst[d].t, want[d], "u32", f"AGV dst[{d}]")
        assert dst[d].guards_ok(), f"AGV dst[{d}] canary"


def test_reduce_scatter_v_128mib(torch, ctx):
    e = 128 * MiB // 4
    c = wl.v_counts(N, e, 1, cfg=wl.CFG_A2A_N8)[0]
    host = [wl.normal_f32(e, wl.CFG_A2A_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    dst = [Out(torch, int(c[r]) * 4) for r in range(N)]
    snac.snac_reduce_scatter_v(ctx, src, [o.t if c[r] else 0 for r, o in enumerate(dst)], c.tolist(), "f32",
                               stream(torch))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter_v(host, c.tolist(), "f32")
    for r in range(N):
        compare_whole(dst[r].t, want[r], "f32", f"RSV dst[{r}]")
        assert dst[r].guards_ok(), f"RSV dst[{r}] canary"


# ------------------------------------------------------- SNAC pipeline
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pipeline_4096x8192(torch, ctx, dtype):
    """Whole output against oracle.pipeline_scale_reduce, in the staging ring
    the benchmark uses (128 MiB per rank), and a repeat run bit-identical."""
    count = 4096 * 8192
    if dtype == "bf16":
        host = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r) for r in range(N)]
    else:
        host = [wl.normal_f32(count, wl.CFG_PIPELINE_N8, r) for r in range(N)]
    xs = [up(torch, h) for h in host]
    es = host[0].itemsize
    out = Out(torch, count * es)
    st = stream(torch)
    pctx = snac.snac_init(N, 128 * MiB, st)
    try:
        snac.snac_pipeline_scale_reduce(pctx, xs, out.t, count, dtype, st)
        snac.snac_check(pctx, st)
        want = oracle.pipeline_scale_reduce(host, dtype)
        compare_whole(out.t, want, dtype, f"pipeline {dtype}")
        assert out.guards_ok(), "pipeline output canary"
        again = Out(torch, count * es)
        snac.snac_pipeline_scale_reduce(pctx, xs, again.t, count, dtype, st)
        snac.snac_check(pctx, st)
        assert torch.equal(again.t, out.t)
    finally:
        snac.snac_finalize(pctx, st)


def test_pipeline_latency_sizes(torch, ctx):
    """The small-message sweep sizes, 1 KiB .. 1 MiB per rank, full check."""
    for p in range(10, 21):
        count = (1 << p) // 2
        host = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r, seed=p) for r in range(N)]
        xs = [up(torch, h) for h in host]
        out = Out(torch, count * 2)
        snac.snac_pipeline_scale_reduce(ctx, xs, out.t, count, "bf16", stream(torch))
        snac.snac_check(ctx, stream(torch))
        assert_same(out.t.cpu().numpy().view(np.uint16), oracle.pipeline_scale_reduce(host, "bf16"), "bf16",
                    f"pipeline {1 << p} B/rank")
        assert out.guards_ok()
