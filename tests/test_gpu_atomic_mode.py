"""The non-deterministic (atomic) AllReduce mode against the mathematics,
since its bits depend on the order the hardware applies the adds:

* within the stated bound of the exact sum: |result - S| <= N * 2^-24 *
  sum_k |x_k| + half an output ulp (binary32 adds from +0.0 in any order,
  then one rounding), with S computed in float64 from the same inputs;
* exact where every partial sum is exact in any order (small integers);
* all N destinations bitwise equal (one rounding, written N times);
* the deterministic mode of the same entry point is the plain AllReduce.
"""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype
from oracle.bf16 import bf16_to_f32, f32_to_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

U = 2.0 ** -24


def sync():
    import torch

    torch.cuda.synchronize()


def as_f64(a, dtype):
    return (bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


def half_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    mant = 7 if dtype == "bf16" else 23
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - mant - 1)


def run_atomic(ctx, srcs, dtype, offset=0):
    nb = srcs[0].nbytes
    sb = [DevBuf(nb, offset=offset, data=s) for s in srcs]
    db = [DevBuf(nb, offset=offset) for _ in srcs]
    snac.snac_all_reduce_ex(ctx, [b.ptr for b in sb], [b.ptr for b in db], nb, dtype, "atomic")
    sync()
    snac.snac_check(ctx)
    for b in db:
        assert b.guards_ok()
    return [b.download(np_dtype(dtype)) for b in db]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [2, 3, 8])
@pytest.mark.parametrize("offset", [0, 4])
def test_atomic_within_bound(dtype, n, offset):
    m = 100_003
    srcs = [wl.normal_bf16(m, wl.CFG_TEST, r, seed=n) if dtype == "bf16" else
            wl.normal_f32(m, wl.CFG_TEST, r, seed=n) for r in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        outs = run_atomic(ctx, srcs, dtype, offset)
    finally:
        snac.snac_finalize(ctx)
    xs = np.stack([as_f64(s, dtype) for s in srcs])
    exact = xs.sum(axis=0)
    bound = n * U * np.abs(xs).sum(axis=0)
    got = as_f64(outs[0], dtype)
    err = np.abs(got - exact)
    lim = bound + half_ulp(exact, dtype) * 1.0000001
    assert np.all(err <= lim), f"worst excess {np.max(err - lim)} at {int(np.argmax(err - lim))}"
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_atomic_exact_on_integers_and_many_chunks(dtype):
    """Integer inputs sum exactly in any order, so the atomic mode must
    equal the oracle bit for bit; a 96 KiB-per-rank staging ring makes the
    accumulator serve the 600_001-element message in several chunks."""
    n, m = 8, 600_001
    i = np.arange(m)
    vals = [((k + 1) * (i % 7)).astype(np.float32) for k in range(n)]
    srcs = [f32_to_bf16(v) for v in vals] if dtype == "bf16" else vals
    ctx = snac.snac_init(n, 96 << 10)
    try:
        outs = run_atomic(ctx, srcs, dtype)
    finally:
        snac.snac_finalize(ctx)
    want = oracle.all_reduce(srcs, dtype)
    for o, w in zip(outs, want):
        assert_same(o, w, dtype, "atomic mode on integers")


def test_deterministic_mode_is_the_plain_allreduce():
    n, m = 8, 77_777
    srcs = [wl.normal_bf16(m, wl.CFG_TEST, r, seed=5) for r in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        sb = [DevBuf(s.nbytes, data=s) for s in srcs]
        db = [DevBuf(s.nbytes) for s in srcs]
        snac.snac_all_reduce_ex(ctx, [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, "bf16",
                                "deterministic")
        sync()
    finally:
        snac.snac_finalize(ctx)
    for b, w in zip(db, oracle.all_reduce(srcs, "bf16")):
        assert_same(b.download(np.uint16), w, "bf16", "deterministic mode")
