"""The allocation-free entry point, snac_all_reduce_atomic_static, against the
entry point it varies: snac_all_reduce_ex in SNAC_REDUCE_ATOMIC mode, both
called through the C ABI.

Two calls in a row, the second with a smaller message, each compared with the
existing entry point's output on the same inputs:

* integer-valued inputs, whose sums are exact in any order of the adds:
  both entry points must agree bit for bit, and with the oracle;
* N(0,1) inputs: the atomic mode's bits depend on the order the hardware
  applies the adds, so each output must lie within the mode's bound of the
  float64 sum, |result - S| <= N * 2^-24 * sum|x| + half an output ulp, and
  the two entry points within twice that of each other;
* every destination equal to destination 0, and the bytes around every
  output (canaries) untouched.

Also: the largest message the static accumulator holds (2^23 elements per
rank) works, one element more is refused before anything is enqueued.
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
MAX_ELEMS = 1 << 23


def sync():
    import torch

    torch.cuda.synchronize()


def as_f64(a, dtype):
    return (bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


def half_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    mant = 7 if dtype == "bf16" else 23
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - mant - 1)


def both(ctx, srcs, dtype, offset=0):
    """(static entry point's outputs, existing atomic entry point's outputs)
    for the same inputs, each into canary-guarded destinations."""
    nb = srcs[0].nbytes
    sb = [DevBuf(nb, offset=offset, data=s) for s in srcs]
    outs = []
    for which in ("static", "ex"):
        db = [DevBuf(nb, offset=offset) for _ in srcs]
        if which == "static":
            snac.snac_all_reduce_atomic_static([b.ptr for b in sb], [b.ptr for b in db], nb, dtype)
        else:
            snac.snac_all_reduce_ex(ctx, [b.ptr for b in sb], [b.ptr for b in db], nb, dtype, "atomic")
        sync()
        for r, b in enumerate(db):
            assert b.guards_ok(), f"{which}: canary around dst[{r}]"
        got = [b.download(np_dtype(dtype)) for b in db]
        for r in range(1, len(got)):
            assert np.array_equal(got[r].view(np.uint8), got[0].view(np.uint8)), f"{which}: dst[{r}] != dst[0]"
        outs.append(got)
    snac.snac_check(ctx)
    return outs


def integer_inputs(n, m, dtype, shift):
    i = np.arange(m)
    vals = [((k + 1 + shift) * ((i + k) % 7)).astype(np.float32) for k in range(n)]
    return [f32_to_bf16(v) for v in vals] if dtype == "bf16" else vals


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_equals_atomic_entry_point_on_integers(dtype):
    n = 8
    ctx = snac.snac_init(n, 0)
    try:
        for m, shift in ((1_000_003, 0), (300_001, 1)):  # the second call smaller
            srcs = integer_inputs(n, m, dtype, shift)
            st, ex = both(ctx, srcs, dtype)
            want = oracle.all_reduce(srcs, dtype)
            for r in range(n):
                assert_same(st[r], ex[r], dtype, f"static vs atomic entry point, m={m}, dst[{r}]")
                assert_same(st[r], want[r], dtype, f"static vs oracle, m={m}, dst[{r}]")
    finally:
        snac.snac_finalize(ctx)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("offset", [0, 4])
def test_static_within_bound_like_atomic_entry_point(dtype, offset):
    n = 8
    ctx = snac.snac_init(n, 0)
    try:
        for m in (777_777, 65_537):  # the second call smaller
            srcs = [wl.normal_bf16(m, wl.CFG_TEST, r, seed=m) if dtype == "bf16" else
                    wl.normal_f32(m, wl.CFG_TEST, r, seed=m) for r in range(n)]
            st, ex = both(ctx, srcs, dtype, offset)
            xs = np.stack([as_f64(s, dtype) for s in srcs])
            exact = xs.sum(axis=0)
            lim = n * U * np.abs(xs).sum(axis=0) + half_ulp(exact, dtype) * 1.0000001
            a, b = as_f64(st[0], dtype), as_f64(ex[0], dtype)
            assert np.all(np.abs(a - exact) <= lim), f"static: worst excess {np.max(np.abs(a - exact) - lim)}"
            assert np.all(np.abs(b - exact) <= lim), f"atomic: worst excess {np.max(np.abs(b - exact) - lim)}"
            assert np.all(np.abs(a - b) <= 2 * lim)
    finally:
        snac.snac_finalize(ctx)


def test_static_largest_message_and_refusal():
    """2^23 f32 elements per rank fill the 32 MiB accumulator exactly; one
    more element is SNAC_E_ARG and the destinations stay untouched."""
    import torch

    n, dtype = 2, "f32"
    srcs = integer_inputs(n, MAX_ELEMS, dtype, 3)
    ctx = snac.snac_init(n, 0)
    try:
        st, ex = both(ctx, srcs, dtype)
        for r in range(n):
            assert_same(st[r], ex[r], dtype, f"largest message dst[{r}]")
    finally:
        snac.snac_finalize(ctx)
    nb = (MAX_ELEMS + 1) * 4
    src = [torch.zeros(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    dst = [torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(n)]
    with pytest.raises(snac.SnacError) as e:
        snac.snac_all_reduce_atomic_static(src, dst, nb, dtype)
    assert e.value.status == snac.SNAC_E_ARG
    assert "static scratch" in str(e.value)
    sync()
    assert all(bool((d == 0xA5).all().item()) for d in dst)
