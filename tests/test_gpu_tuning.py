"""Tuning rules and the autotuner on the GPU: any launch shape the rules
select leaves every result bit-exact against the oracle, and the autotuner
runs end to end and installs a table the library accepts."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

U64MAX = 2 ** 64 - 1


def sync():
    import torch

    torch.cuda.synchronize()


@pytest.fixture()
def ctx8():
    c = snac.snac_init(8, 0)
    yield c
    snac.snac_finalize(c)
    snac.snac_set_tuning_rules(None)


@pytest.mark.parametrize("wpc,cp", [(4, 4), (3, 2), (1, 3), (8, 1)])
def test_rules_keep_results_exact(ctx8, wpc, cp):
    snac.snac_set_tuning_rules([{"coll": snac.SNAC_RULE_ANY, "min_ranks": 1, "max_ranks": 16, "esize": 0,
                                 "min_bytes": 0, "max_bytes": U64MAX, "wgs_per_cu": wpc, "cache_policy": cp}])
    n, m = 8, 8 * 30_011
    for dtype in ("bf16", "f32"):
        srcs = [wl.normal_bf16(m, wl.CFG_TEST, r, seed=wpc) if dtype == "bf16" else
                wl.uniform_f32(m, wl.CFG_TEST, r, seed=wpc) for r in range(n)]
        sb = [DevBuf(s.nbytes, data=s) for s in srcs]
        db = [DevBuf(s.nbytes) for s in srcs]
        snac.snac_all_reduce(ctx8, [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, dtype)
        e = 2 if dtype == "bf16" else 4
        rb = [DevBuf(s.nbytes // n, offset=e) for s in srcs]  # misaligned: the generic kernels
        snac.snac_reduce_scatter(ctx8, [b.ptr for b in sb], [b.ptr for b in rb], srcs[0].nbytes, dtype)
        sync()
        for b, w in zip(db, oracle.all_reduce(srcs, dtype)):
            assert_same(b.download(np_dtype(dtype)), w, dtype, f"AR wpc={wpc} cp={cp}")
        for b, w in zip(rb, oracle.reduce_scatter(srcs, dtype)):
            assert b.guards_ok()
            assert_same(b.download(np_dtype(dtype)), w, dtype, f"RS wpc={wpc} cp={cp}")
    srcs = [wl.raw_u32(m // n, wl.CFG_TEST, r, seed=wpc) for r in range(n)]
    sb = [DevBuf(s.nbytes, data=s) for s in srcs]
    db = [DevBuf(s.nbytes * n) for s in srcs]
    snac.snac_all_gather(ctx8, [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, "u32")
    sync()
    for b, w in zip(db, oracle.all_gather(srcs)):
        assert_same(b.download(np.uint32), w, "u32", f"AG wpc={wpc} cp={cp}")


def test_autotune_small_sizes_installs_a_table(ctx8):
    from copy_reduce_snac_amd import autotune

    lines = []
    rules = autotune.measure([64 << 10, 1 << 20], steps=3, log=lines.append)
    assert len(lines) == 10  # five workloads at two sizes
    named = [r for r in rules if r["coll"] in (snac.SNAC_COLL_ALL_REDUCE, snac.SNAC_RULE_ATOM_COPY)]
    assert len(named) == 4
    snac.snac_set_tuning_rules(rules)
    assert snac.snac_get_tuning_rules() == rules
    # buckets meet: every size from 0 up is covered exactly once per workload
    ar = sorted((r["min_bytes"], r["max_bytes"]) for r in rules if r["coll"] == snac.SNAC_COLL_ALL_REDUCE)
    assert ar[0][0] == 0 and ar[-1][1] == U64MAX and ar[0][1] + 1 == ar[1][0]
    # and the library still computes the right thing with them
    n, m = 8, 100_000
    srcs = [wl.normal_bf16(m, wl.CFG_TEST, r, seed=77) for r in range(n)]
    sb = [DevBuf(s.nbytes, data=s) for s in srcs]
    db = [DevBuf(s.nbytes) for s in srcs]
    snac.snac_all_reduce(ctx8, [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, "bf16")
    sync()
    for b, w in zip(db, oracle.all_reduce(srcs, "bf16")):
        assert_same(b.download(np.uint16), w, "bf16", "AR under the autotuned table")
