"""Randomised parity of the SNAC pipeline (snac_pipeline_scale_reduce).

Each seeded case draws a rank count, data type, message size, staging ring
size, and optionally a fixed pipeline tile, lookahead and workgroups per CU.
It then runs the call twice on a fresh context, the second time with other
inputs, and compares both outputs with the oracle.  The ring is re-cut per
call (split, merged or compacted slots; one queue or several), and
consumers may trail producers by anything from one tile to the whole ring.
Waits are bounded, so a protocol error shows as a reported status, not a
hang.
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

KiB, MiB = 1 << 10, 1 << 20


def case(i: int):
    rng = np.random.default_rng([20261203, i])
    n = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    dtype = str(rng.choice(["bf16", "f32"]))
    e = 2 if dtype == "bf16" else 4
    ring = int(rng.choice([64 * KiB, 256 * KiB, 1 * MiB, 4 * MiB, 16 * MiB]))
    # a fixed tile (one that divides the ring into at least 2 slots) in a third of the cases
    tile = 0
    if rng.random() < 1 / 3:
        choices = [t for t in (4 * KiB, 8 * KiB, 12 * KiB, 16 * KiB, 64 * KiB, 256 * KiB) if ring % t == 0 and ring // t >= 2]
        tile = int(rng.choice(choices))
    lookahead = int(rng.choice([0, 0, 1, 2, 3, 7]))
    wgs = int(rng.choice([0, 0, 1, 2, 4]))
    # message: from a few elements to several times the ring
    kind = rng.random()
    if kind < 0.3:
        count = int(rng.integers(1, 4096))
    elif kind < 0.7:
        count = int(rng.integers(4096, 2 * MiB // e))
    else:
        count = int(rng.integers(2 * MiB // e, 12 * MiB // e))
    return n, dtype, ring, tile, lookahead, wgs, count, i


# SNAC_RANDOM_PIPELINE_CASES widens the sweep
CASES = [case(i) for i in range(int(os.environ.get("SNAC_RANDOM_PIPELINE_CASES", "24")))]


@pytest.mark.parametrize("n,dtype,ring,tile,lookahead,wgs,count,seed", CASES,
                         ids=[f"n{c[0]}-{c[1]}-ring{c[2]}-tile{c[3]}-la{c[4]}-w{c[5]}-c{c[6]}" for c in CASES])
def test_random_pipeline(n, dtype, ring, tile, lookahead, wgs, count, seed):
    import torch

    t0 = snac.snac_get_tuning()
    try:
        snac.snac_set_tuning(pipeline_tile_bytes=tile, pipeline_lookahead=lookahead, wgs_per_cu=wgs)
        ctx = snac.snac_init(n, ring)
        try:
            for rep in range(2):
                gen = wl.normal_bf16 if dtype == "bf16" else wl.normal_f32
                xs = [gen(count, wl.CFG_TEST, r, seed=seed * 2 + rep) for r in range(n)]
                xb = [DevBuf(x.nbytes, data=x) for x in xs]
                ob = DevBuf(xs[0].nbytes)
                snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in xb], ob.ptr, count, dtype)
                snac.snac_check(ctx)
                torch.cuda.synchronize()
                what = f"pipeline case {seed} rep {rep}: N={n} {dtype} ring={ring} tile={tile} " \
                       f"lookahead={lookahead} wgs={wgs} count={count}"
                assert ob.guards_ok(), what
                assert_same(ob.download(np_dtype(dtype)), oracle.pipeline_scale_reduce(xs, dtype), dtype, what)
        finally:
            snac.snac_finalize(ctx)
    finally:
        snac.snac_set_tuning(**t0)
