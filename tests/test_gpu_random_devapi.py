"""Randomised parity of the device-side collective (snac::collective with
snac_args, include/snac_device.hpp), run by part of a user grid.

Each seeded case draws a collective, rank count, data type, size, buffer
offsets and launch shape: `blocks` workgroups that enter the call, the first
`coll_blocks` of them moving data, and `extra` workgroups of the same grid
that do not take part.  Outputs are compared with the oracle; every
participant must report the collective complete, and no other workgroup
may.  Launch shapes that would not be co-resident are skipped by the
launcher (the closing barrier needs co-residency).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEVLIB = os.path.join(os.path.dirname(__file__), "devapi", "libsnac_devtest.so")
_VP, _I = ctypes.c_void_p, ctypes.c_int
_DP = ctypes.POINTER(snac.snac_coll_desc)
_CP = ctypes.POINTER(snac.snac_dev_ctx)
ESIZE = {"bf16": 2, "f32": 4, "u32": 4, "byte": 1}
COLLS = [snac.SNAC_COLL_ALL_REDUCE, snac.SNAC_COLL_REDUCE_SCATTER, snac.SNAC_COLL_ALL_GATHER,
         snac.SNAC_COLL_ALL_TO_ALL, snac.SNAC_COLL_ALL_GATHER_V, snac.SNAC_COLL_REDUCE_SCATTER_V,
         snac.SNAC_COLL_ALL_TO_ALL_V]
REDUCES = {snac.SNAC_COLL_ALL_REDUCE, snac.SNAC_COLL_REDUCE_SCATTER, snac.SNAC_COLL_REDUCE_SCATTER_V}


def gen(n, m, dtype, seed):
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "u32":
        return [wl.raw_u32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


def case(i: int):
    rng = np.random.default_rng([20261204, i])
    coll = COLLS[i % len(COLLS)]
    n = int(rng.choice([1, 2, 3, 4, 8, 16]))  # the rank counts the test kernels are built for
    dtype = str(rng.choice(["bf16", "f32"] if coll in REDUCES else ["bf16", "u32", "byte"]))
    e = ESIZE[dtype]
    m = int(rng.integers(1, (3 << 20) // e))
    if coll in (snac.SNAC_COLL_REDUCE_SCATTER, snac.SNAC_COLL_ALL_TO_ALL):
        m = max(n, m - m % n)
    if coll == snac.SNAC_COLL_ALL_GATHER:
        m = max(1, m // n)
    blocks = int(rng.choice([1, 2, 7, 32, 64, 128, 240]))  # with extra, at most 256: one per CU always fits
    coll_blocks = int(rng.integers(1, blocks + 1))
    extra = int(rng.choice([0, 0, 3, 16]))
    offs = [int(o) for o in rng.integers(0, 16, size=2 * n) * e]
    return coll, n, dtype, m, blocks, coll_blocks, extra, offs, i


CASES = [case(i) for i in range(int(os.environ.get("SNAC_RANDOM_DEVAPI_CASES", "21")))]


@pytest.fixture(scope="module")
def dev():
    if not os.path.exists(DEVLIB):
        raise RuntimeError(f"{DEVLIB} missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(DEVLIB)
    lib.devtest_collective.argtypes = [_DP, _CP, _I, _I, _I, _I, _I, _I, _VP, _VP]
    lib.devtest_collective.restype = _I
    return lib


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


@pytest.mark.parametrize("coll,n,dtype,m,blocks,coll_blocks,extra,offs,seed", CASES,
                         ids=[f"c{c[0]}-n{c[1]}-{c[2]}-m{c[3]}-b{c[4]}-{c[5]}-{c[6]}" for c in CASES])
def test_random_device_collective(dev, ctxs, coll, n, dtype, m, blocks, coll_blocks, extra, offs, seed):
    import torch

    counts = None
    if coll in (snac.SNAC_COLL_ALL_GATHER_V, snac.SNAC_COLL_REDUCE_SCATTER_V):
        counts = [int(c) for c in wl.v_counts(n, m, 1, cfg=wl.CFG_TEST, seed=seed)[0]]
    elif coll == snac.SNAC_COLL_ALL_TO_ALL_V:
        counts = wl.v_counts(n, m, n, cfg=wl.CFG_TEST, seed=seed)
    ins = counts if coll == snac.SNAC_COLL_ALL_GATHER_V else [m] * n
    xs = [x[:k] for x, k in zip(gen(n, max(ins), dtype, seed), ins)]
    if coll == snac.SNAC_COLL_ALL_REDUCE:
        want = oracle.all_reduce(xs, dtype)
    elif coll == snac.SNAC_COLL_REDUCE_SCATTER:
        want = oracle.reduce_scatter(xs, dtype)
    elif coll == snac.SNAC_COLL_ALL_GATHER:
        want = oracle.all_gather(xs)
    elif coll == snac.SNAC_COLL_ALL_TO_ALL:
        want = oracle.all_to_all(xs)
    elif coll == snac.SNAC_COLL_ALL_GATHER_V:
        want = oracle.all_gather_v(xs, counts)
    elif coll == snac.SNAC_COLL_REDUCE_SCATTER_V:
        want = oracle.reduce_scatter_v(xs, counts, dtype)
    else:
        want = oracle.all_to_all_v(xs, counts)
    sb = [DevBuf(x.nbytes, offset=o, data=x) for x, o in zip(xs, offs[:n])]
    db = [DevBuf(np.asarray(w).nbytes, offset=o) for w, o in zip(want, offs[n:])]
    flat = None if counts is None else np.asarray(counts).reshape(-1).tolist()
    ctx = ctxs(n)
    desc = snac.snac_describe(ctx, coll, [b.ptr for b in sb], [b.ptr for b in db], m * ESIZE[dtype], flat, dtype)
    dctx = snac.snac_get_device_context(ctx)
    ok = torch.zeros(blocks + extra, dtype=torch.int32, device="cuda")
    rc = dev.devtest_collective(ctypes.byref(desc), ctypes.byref(dctx), int(dtype == "bf16"), n, blocks, coll_blocks,
                                extra, 0, ok.data_ptr(), None)
    if rc == -1:
        pytest.skip(f"{blocks + extra} workgroups are not co-resident")
    assert rc == 0, f"launcher returned {rc}"
    torch.cuda.synchronize()
    snac.snac_check(ctx)
    what = f"device collective {coll} N={n} {dtype} m={m} blocks={blocks}/{coll_blocks}+{extra} case {seed}"
    assert ok[:blocks].cpu().numpy().tolist() == [1] * blocks, what
    assert ok[blocks:].cpu().numpy().tolist() == [0] * extra, what
    for r, (b, w) in enumerate(zip(db, want)):
        assert b.guards_ok(), f"{what}: canary overwritten around dst[{r}]"
        assert_same(b.download(np_dtype(dtype)), np.asarray(w), dtype, f"{what} dst[{r}]")
