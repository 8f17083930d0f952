"""Brute force over small shapes on the GPU: every collective for N in
{1, 2, 3, 4, 8}, element counts from 0 to 256 and random element-aligned
byte offsets 0..15 of every buffer, V counts with zeros, all bit-exact
against the oracle with canaries intact."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SIZES = [0, 1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 200, 255, 256]


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


def gen(n, m, dtype, seed):
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "u32":
        return [wl.raw_u32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


def offsets(rng, n, e):
    return [int(rng.integers(0, 16 // e)) * e for _ in range(n)]


def check(dbs, wants, dtype, what):
    import torch

    torch.cuda.synchronize()
    for r, (b, w) in enumerate(zip(dbs, wants)):
        assert b.guards_ok(), f"{what}: canary around dst[{r}]"
        assert_same(b.download(np_dtype(dtype)), np.asarray(w), dtype, f"{what} dst[{r}]")


CASES = [("all_reduce", "bf16"), ("all_reduce", "f32"), ("reduce_scatter", "bf16"), ("all_gather", "byte"),
         ("all_to_all", "u32"), ("all_gather_v", "bf16"), ("reduce_scatter_v", "f32"), ("all_to_all_v", "byte")]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("coll,dtype", CASES)
def test_bruteforce(ctxs, coll, dtype, n):
    rng = np.random.default_rng(hash((coll, dtype, n)) % (1 << 32))
    e = np.dtype(np_dtype(dtype)).itemsize
    ctx = ctxs(n)
    for size in SIZES:
        seed = size * 31 + n
        so, do = offsets(rng, n, e), offsets(rng, n, e)
        what = f"{coll} {dtype} N={n} size={size} src_off={so} dst_off={do}"
        if coll in ("all_reduce", "reduce_scatter", "all_gather", "all_to_all"):
            m = size - size % n if coll in ("reduce_scatter", "all_to_all") else size
            srcs = gen(n, m, dtype, seed)
            want = {"all_reduce": lambda: oracle.all_reduce(srcs, dtype),
                    "reduce_scatter": lambda: oracle.reduce_scatter(srcs, dtype),
                    "all_gather": lambda: oracle.all_gather(srcs),
                    "all_to_all": lambda: oracle.all_to_all(srcs)}[coll]()
            sb = [DevBuf(s.nbytes, offset=so[k], data=s) for k, s in enumerate(srcs)]
            db = [DevBuf(np.asarray(w).nbytes, offset=do[k]) for k, w in enumerate(want)]
            getattr(snac, "snac_" + coll)(ctx, [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, dtype)
            check(db, want, dtype, what)
            continue
        if coll == "all_to_all_v":
            c = wl.v_counts(n, size, n, cfg=wl.CFG_TEST, seed=seed)
            srcs = gen(n, size, dtype, seed)
            want = oracle.all_to_all_v(srcs, c)
            counts = c.reshape(-1).tolist()
        else:
            row = [int(x) for x in wl.v_counts(n, size, 1, cfg=wl.CFG_TEST, seed=seed)[0]]
            counts = row
            if coll == "all_gather_v":
                srcs = [gen(1, row[k], dtype, seed + k)[0] for k in range(n)]
                want = oracle.all_gather_v(srcs, row)
            else:
                srcs = gen(n, size, dtype, seed)
                want = oracle.reduce_scatter_v(srcs, row, dtype)
        sb = [DevBuf(s.nbytes, offset=so[k], data=s) for k, s in enumerate(srcs)]
        db = [DevBuf(np.asarray(w).nbytes, offset=do[k]) for k, w in enumerate(want)]
        getattr(snac, "snac_" + coll)(ctx, [b.ptr for b in sb], [b.ptr for b in db], counts, dtype)
        check(db, want, dtype, what + f" counts={counts}")
