"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (library defaults).  The oracle computes a seeded sample of
output positions one by one (2^16 random positions plus the first and last
4096 of every output); properties that hold at any size (AllGather of
ReduceScatter equals AllReduce bit for bit, repeat runs are identical) are
checked on the whole output on the GPU."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import assert_same, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MiB = 1 << 20
N = 8


@pytest.fixture(scope="module")
def torch():
    import torch

    torch.cuda.set_device(0)
    return torch


@pytest.fixture(scope="module")
def ctx(torch):
    c = snac.snac_init(N, 0)
    yield c
    snac.snac_finalize(c)


def up(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).cuda()


def sample_idx(m: int, seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(min(4096, m)), np.arange(max(0, m - 4096), m)])
    return np.unique(np.concatenate([edge, g.integers(0, m, size=min(1 << 16, m))]))


def gather(torch, t, idx: np.ndarray, np_dtype):
    """Elements idx of the device byte tensor t viewed as np_dtype."""
    tdt = {np.uint16: torch.int16, np.float32: torch.float32, np.uint32: torch.int32}[np_dtype]
    v = t.view(tdt)[torch.from_numpy(idx.astype(np.int64)).cuda()]
    return v.cpu().numpy().view(np_dtype)


def test_allreduce_bf16_n8_256mib(torch, ctx):
    per_rank = 256 * MiB
    m = per_rank // 2
    host = [wl.normal_bf16(m, wl.CFG_AR_BF16_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    dst = [torch.empty(per_rank, dtype=torch.uint8, device="cuda") for _ in range(N)]
    snac.snac_all_reduce(ctx, src, dst, per_rank, "bf16")
    torch.cuda.synchronize()
    idx = sample_idx(m, 1)
    want = oracle.reduce_n([h[idx] for h in host], "bf16")
    for r in range(N):
        assert_same(gather(torch, dst[r], idx, np.uint16), want, "bf16", f"AR 256MiB dst[{r}]")
        if r:
            assert torch.equal(dst[r], dst[0])
    # repeat run: bit-identical (deterministic mode)
    again = [torch.empty_like(d) for d in dst]
    snac.snac_all_reduce(ctx, src, again, per_rank, "bf16")
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(again, dst))


def test_allreduce_bf16_n8_size_sweep(torch, ctx):
    """Per-rank sizes 1 KiB .. 64 MiB (powers of two), full comparison."""
    top = 64 * MiB
    host = [wl.normal_bf16(top // 2, wl.CFG_AR_BF16_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    dst = [torch.empty(top, dtype=torch.uint8, device="cuda") for _ in range(N)]
    for p in range(10, 27, 2):
        b = 1 << p
        snac.snac_all_reduce(ctx, src, dst, b, "bf16")
        torch.cuda.synchronize()
        want = oracle.reduce_n([h[: b // 2] for h in host], "bf16")
        got = dst[N - 1][:b].cpu().numpy().view(np.uint16)
        assert_same(got, want, "bf16", f"AR {b} B/rank")


def test_rs_then_ag_equals_allreduce(torch, ctx):
    rows, cols = N * 4096, 2048
    m = rows * cols
    per_rank = m * 2
    host = [wl.normal_bf16(m, wl.CFG_RS_AG_BF16_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    rs = [torch.empty(per_rank // N, dtype=torch.uint8, device="cuda") for _ in range(N)]
    ag = [torch.empty(per_rank, dtype=torch.uint8, device="cuda") for _ in range(N)]
    ar = [torch.empty(per_rank, dtype=torch.uint8, device="cuda") for _ in range(N)]
    snac.snac_reduce_scatter(ctx, src, rs, per_rank, "bf16")
    snac.snac_all_gather(ctx, rs, ag, per_rank // N, "bf16")
    snac.snac_all_reduce(ctx, src, ar, per_rank, "bf16")
    torch.cuda.synchronize()
    for r in range(N):
        assert torch.equal(ag[r], ar[r]), f"AG(RS(x))[{r}] != AR(x)[{r}]"
    idx = sample_idx(m, 2)
    want = oracle.reduce_n([h[idx] for h in host], "bf16")
    assert_same(gather(torch, ag[3], idx, np.uint16), want, "bf16", "RS->AG sampled")
    # chunk r of the ReduceScatter output sits on rank r
    mc = m // N
    for r in (0, N - 1):
        ridx = sample_idx(mc, 3 + r)
        want = oracle.reduce_n([h[r * mc + ridx] for h in host], "bf16")
        assert_same(gather(torch, rs[r], ridx, np.uint16), want, "bf16", f"RS chunk {r}")


@pytest.mark.parametrize("dtype", ["u32", "f32"])
def test_all_to_all_128mib(torch, ctx, dtype):
    e = 128 * MiB // 4
    host = [wl.raw_u32(e, wl.CFG_A2A_N8, r) if dtype == "u32" else wl.uniform_f32(e, wl.CFG_A2A_N8, r)
            for r in range(N)]
    npd = np.uint32 if dtype == "u32" else np.float32
    src = [up(torch, h) for h in host]
    dst = [torch.empty(e * 4, dtype=torch.uint8, device="cuda") for _ in range(N)]
    snac.snac_all_to_all(ctx, src, dst, e * 4, dtype)
    torch.cuda.synchronize()
    mc = e // N
    g = np.random.default_rng(4)
    for d in range(N):
        idx = sample_idx(e, 10 + d)
        s = idx // mc
        i = idx % mc
        want = np.array([host[int(ss)][d * mc + int(ii)] for ss, ii in zip(s, i)], dtype=npd)
        got = gather(torch, dst[d], idx, npd)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"A2A dst[{d}]"


def _v_check(torch, dst, wants_fn, sizes, npd, what):
    for d, t in enumerate(dst):
        if sizes[d] == 0:
            continue
        idx = sample_idx(sizes[d], 20 + d)
        want = wants_fn(d, idx)
        got = gather(torch, t, idx, npd)
        assert np.array_equal(got.view(np.uint32), np.asarray(want).view(np.uint32)), f"{what} dst[{d}]"


def test_all_to_all_v_128mib(torch, ctx):
    e = 128 * MiB // 4
    c = wl.v_counts(N, e, N, cfg=wl.CFG_A2A_N8)
    assert (c == 0).any() and (c % 4 != 0).any()
    host = [wl.raw_u32(e, wl.CFG_A2A_N8, r) for r in range(N)]
    src = [up(torch, h) for h in host]
    cols = c.sum(axis=0)
    dst = [torch.empty(max(1, int(cols[d])) * 4, dtype=torch.uint8, device="cuda") for d in range(N)]
    snac.snac_all_to_all_v(ctx, src, dst, c.reshape(-1).tolist(), "u32")
    torch.cuda.synchronize()
    sd = np.concatenate([np.zeros((N, 1), np.int64), np.cumsum(c, axis=1)[:, :-1]], axis=1)  # send displ
    rd = np.concatenate([np.zeros((1, N), np.int64), np.cumsum(c, axis=0)[:-1, :]], axis=0)  # recv displ

    def want(d, idx):
        out = np.empty(len(idx), dtype=np.uint32)
        for k, i in enumerate(idx):
            s = int(np.searchsorted(rd[:, d], i, side="right") - 1)
            while c[s, d] == 0 or i >= rd[s, d] + c[s, d]:
                s += 1
            out[k] = host[s][sd[s, d] + (i - rd[s, d])]
        return out

    _v_check(torch, dst, want, [int(x) for x in cols], np.uint32, "A2AV")


def test_all_gather_v_and_reduce_scatter_v(torch, ctx):
    e = 128 * MiB // 4
    c = wl.v_counts(N, e, 1, cfg=wl.CFG_A2A_N8)[0]
    disp = np.concatenate([[0], np.cumsum(c)[:-1]])
    host = [wl.raw_u32(int(c[k]), wl.CFG_A2A_N8, k) for k in range(N)]
    src = [up(torch, h) if h.size else torch.empty(0, dtype=torch.uint8, device="cuda") for h in host]
    dst = [torch.empty(e * 4, dtype=torch.uint8, device="cuda") for _ in range(N)]
    snac.snac_all_gather_v(ctx, src, dst, c.tolist(), "u32")
    torch.cuda.synchronize()

    def want_agv(d, idx):
        k = np.searchsorted(disp, idx, side="right") - 1
        return np.array([host[int(kk)][int(i - disp[kk])] for kk, i in zip(k, idx)], dtype=np.uint32)

    _v_check(torch, dst, want_agv, [e] * N, np.uint32, "AGV")
    for r in range(1, N):
        assert torch.equal(dst[r], dst[0])
    del src, dst
    fhost = [wl.normal_f32(e, wl.CFG_A2A_N8, r) for r in range(N)]
    fsrc = [up(torch, h) for h in fhost]
    rdst = [torch.empty(max(1, int(c[r])) * 4, dtype=torch.uint8, device="cuda") for r in range(N)]
    snac.snac_reduce_scatter_v(ctx, fsrc, rdst, c.tolist(), "f32")
    torch.cuda.synchronize()

    def want_rsv(r, idx):
        return oracle.reduce_n([h[disp[r] + idx] for h in fhost], "f32")

    _v_check(torch, rdst, want_rsv, [int(x) for x in c], np.float32, "RSV")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pipeline_4096x8192(torch, ctx, dtype):
    count = 4096 * 8192
    if dtype == "bf16":
        host = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r) for r in range(N)]
        npd = np.uint16
    else:
        host = [wl.normal_f32(count, wl.CFG_PIPELINE_N8, r) for r in range(N)]
        npd = np.float32
    xs = [up(torch, h) for h in host]
    out = torch.empty(count * host[0].itemsize, dtype=torch.uint8, device="cuda")
    snac.snac_pipeline_scale_reduce(ctx, xs, out, count, dtype)
    snac.snac_check(ctx)
    idx = sample_idx(count, 5)
    want = oracle.pipeline_scale_reduce([h[idx] for h in host], dtype)
    assert_same(gather(torch, out, idx, npd), want, dtype, f"pipeline {dtype}")
    again = torch.empty_like(out)
    snac.snac_pipeline_scale_reduce(ctx, xs, again, count, dtype)
    snac.snac_check(ctx)
    assert torch.equal(again, out)


def test_pipeline_latency_sizes(torch, ctx):
    """The small-message sweep sizes, 1 KiB .. 1 MiB per rank, full check."""
    for p in range(10, 21):
        count = (1 << p) // 2
        host = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r, seed=p) for r in range(N)]
        xs = [up(torch, h) for h in host]
        out = torch.empty(count * 2, dtype=torch.uint8, device="cuda")
        snac.snac_pipeline_scale_reduce(ctx, xs, out, count, "bf16")
        snac.snac_check(ctx)
        assert_same(out.cpu().numpy().view(np.uint16), oracle.pipeline_scale_reduce(host, "bf16"), "bf16",
                    f"pipeline {1 << p} B/rank")
