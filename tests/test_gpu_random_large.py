"""Randomised parity at sizes that run the 16 KiB-tile kernels.

Every collective, rank counts of 2 to 16, the data types each accepts, and
per-rank sizes of several MiB that are not multiples of a tile, so that each
message has more 16 KiB tiles than the GPU has CUs.  Every source and
destination buffer sits at its own element offset from a 256-byte boundary:
jobs then take the generic path, with heads up to the destination's next
128-byte line, leads up to its 16 KiB grid, tails, and loads from sources
that are not aligned like their destinations.  V counts come from the
Dirichlet generator with zero-length chunks.  Whole outputs are compared with
the oracle, and the canaries around every buffer are checked.  Cases are
seeded, so a failure names a case that can be run again on its own.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MiB = 1 << 20
ESIZE = {"bf16": 2, "f32": 4, "u32": 4, "byte": 1}
COLLS = ["all_reduce", "reduce_scatter", "all_gather", "all_to_all", "all_gather_v", "reduce_scatter_v",
         "all_to_all_v"]
REDUCES = {"all_reduce", "reduce_scatter", "reduce_scatter_v"}


def gen(n, m, dtype, seed):
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "u32":
        return [wl.raw_u32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


GRID_COLLS = ["all_reduce", "reduce_scatter", "all_gather", "all_to_all"]


def case(i: int, grid: bool = False):
    """Case i: collective, rank count, data type, sizes and buffer offsets.
    grid: every buffer and size on the 16-byte grid (the aligned kernels),
    sizes still ragged against the 16 KiB tile; every other AllReduce case
    is bf16 over 8 ranks, which has a kernel of its own."""
    rng = np.random.default_rng([20261202, 1, i] if grid else [20261202, i])
    colls = GRID_COLLS if grid else COLLS
    coll = colls[i % len(colls)]
    n = int(rng.choice([2, 3, 5, 8, 16]))
    dtype = str(rng.choice(["bf16", "f32"] if coll in REDUCES else ["bf16", "u32", "byte"]))
    if grid and coll == "all_reduce" and (i // len(colls)) % 2 == 0:
        n, dtype = 8, "bf16"
    e = ESIZE[dtype]
    unit = 16 // e if grid else 1

    def elems(lo_bytes, hi_bytes, multiple=1):
        multiple = int(np.lcm(multiple, unit))
        m = int(rng.integers(lo_bytes // e, hi_bytes // e))
        m -= m % multiple
        return max(m, multiple)

    if coll in ("all_reduce", "reduce_scatter"):
        m = elems(5 * MiB, 12 * MiB, n if coll == "reduce_scatter" else 1)
        if grid and coll == "reduce_scatter":
            m = elems(5 * MiB, 12 * MiB, n * unit)  # each rank's chunk on the grid too
    elif coll == "all_gather":
        # N jobs of m elements; the output holds N * N * m
        m = elems(max(5 * MiB // n, 64 << 10), max(256 * MiB // (n * n), 6 * MiB // n))
    elif coll == "all_to_all":
        m = elems(max(5 * MiB // n, 64 << 10), 12 * MiB, n * unit if grid else n)
    else:
        m = elems(5 * MiB, 16 * MiB)  # per-rank total of the V counts
    offs = rng.integers(0, 16, size=2 * n) * (16 if grid else e)
    return coll, n, dtype, m, [int(o) for o in offs[:n]], [int(o) for o in offs[n:]], i


# SNAC_RANDOM_LARGE_CASES widens the sweep (the default covers each collective four times);
# SNAC_RANDOM_GRID_CASES the one on the 16-byte grid (default: each of its collectives three times)
CASES = [case(i) for i in range(int(os.environ.get("SNAC_RANDOM_LARGE_CASES", "28")))]
CASES += [case(i, grid=True)[:-1] + (1000 + i,)
          for i in range(int(os.environ.get("SNAC_RANDOM_GRID_CASES", "12")))]


@pytest.fixture(scope="module")
def ctxs():
    made = {}

    def get(n):
        if n not in made:
            made[n] = snac.snac_init(n, 0)
        return made[n]

    yield get
    for c in made.values():
        snac.snac_finalize(c)


@pytest.mark.parametrize("coll,n,dtype,m,src_offs,dst_offs,seed", CASES,
                         ids=[f"{c[0]}-n{c[1]}-{c[2]}-{c[3]}" for c in CASES])
def test_random_large(ctxs, coll, n, dtype, m, src_offs, dst_offs, seed):
    import torch

    e = ESIZE[dtype]
    ctx = ctxs(n)
    if coll == "all_gather_v" or coll == "reduce_scatter_v":
        counts = [int(c) for c in wl.v_counts(n, m, 1, cfg=wl.CFG_TEST, seed=seed)[0]]
    elif coll == "all_to_all_v":
        C = wl.v_counts(n, m, n, cfg=wl.CFG_TEST, seed=seed)
    # per-rank input elements
    if coll == "all_gather_v":
        ins = counts
    else:
        ins = [m] * n
    xs = [x[:k] for x, k in zip(gen(n, max(ins), dtype, seed), ins)]
    src = [DevBuf(x.nbytes, offset=o, data=x) for x, o in zip(xs, src_offs)]
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
        want = oracle.all_to_all_v(xs, C)
    dst = [DevBuf(np.asarray(w).nbytes, offset=o) for w, o in zip(want, dst_offs)]
    sp, dp = [b.ptr for b in src], [b.ptr for b in dst]
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
        snac.snac_all_to_all_v(ctx, sp, dp, C.reshape(-1).tolist(), dtype)
    torch.cuda.synchronize()
    what = f"{coll} N={n} {dtype} m={m} case {seed}"
    for r, (b, w) in enumerate(zip(dst, want)):
        assert b.guards_ok(), f"{what}: canary overwritten around dst[{r}]"
        assert_same(b.download(np_dtype(dtype)), np.asarray(w), dtype, f"{what} dst[{r}]")
    for r, b in enumerate(src):
        assert b.guards_ok(), f"{what}: canary overwritten around src[{r}]"
