"""GPU parity of the device-side API (include/snac_device.hpp) against the
CPU oracle: kernels in tests/devapi/devapi_kernels.hip call the workgroup
Atoms, run described collectives on a subset of their grid, and fuse
compute, an in-kernel AllReduce and a read of its result into one kernel.
Bit-exact comparisons; destinations are canary-guarded."""
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
_VP, _I, _U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
_DP = ctypes.POINTER(snac.snac_coll_desc)
_CP = ctypes.POINTER(snac.snac_dev_ctx)


@pytest.fixture(scope="module")
def dev():
    if not os.path.exists(DEVLIB):
        raise RuntimeError(f"{DEVLIB} missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(DEVLIB)
    sigs = {
        "devtest_copy_slices": [_VP, _VP, _U64, _I, _VP],
        "devtest_reduce_slices": [_DP, _I, _U64, _I, _I, _VP],
        "devtest_collective": [_DP, _CP, _I, _I, _I, _I, _I, _I, _VP, _VP],
        "devtest_collective_nosync": [_DP, _CP, _I, _I, _I, _VP, _VP],
        "devtest_fused_scale_allreduce": [_DP, _CP, _DP, _U64, _VP, _I, _VP, _VP],
        "devtest_flags": [_CP, _DP, _VP, _VP, _I, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, _U64, _VP,
                          _VP],
        "devtest_many_flags": [_CP, _VP, _I, _U64, _VP, _VP, _VP],
        "devtest_atom_contract": [_VP],
        "devtest_static_lds": [_I, _VP],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = _I
    return lib


@pytest.fixture(scope="module")
def ctx8():
    c = snac.snac_init(8, 0)
    yield c
    snac.snac_finalize(c)


def sync():
    import torch

    torch.cuda.synchronize()


def ok_buffer(n):
    import torch

    return torch.zeros(n, dtype=torch.int32, device="cuda")


def launch(rc):
    assert rc == 0, f"launcher returned {rc}"


def gen(n, m, dtype, seed):
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "u32":
        return [wl.raw_u32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


# ------------------------------------------------------- workgroup Atoms
@pytest.mark.parametrize("dst_off,src_off", [(0, 0), (1, 3), (7, 2), (16, 5), (3, 3)])
def test_copy_slices_any_alignment(dev, dst_off, src_off):
    blocks, per = 37, 10_007
    src = wl.raw_bytes(blocks * per, wl.CFG_TEST, 0, seed=dst_off * 31 + src_off)
    sb = DevBuf(src.nbytes, offset=src_off, data=src)
    db = DevBuf(src.nbytes, offset=dst_off)
    launch(dev.devtest_copy_slices(db.ptr, sb.ptr, per, blocks, None))
    sync()
    assert db.guards_ok()
    assert_same(db.download(), oracle.copy(src), "byte", "snac::copy slices")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nsrc,ndst", [(1, 1), (2, 3), (3, 1), (8, 2), (16, 1)])
def test_reduce_slices(dev, dtype, nsrc, ndst):
    e = 2 if dtype == "bf16" else 4
    blocks, per = 19, 5003
    srcs = gen(nsrc, blocks * per, dtype, seed=nsrc * 7 + ndst)
    sb = [DevBuf(s.nbytes, offset=e * (k % 5), data=s) for k, s in enumerate(srcs)]
    db = [DevBuf(srcs[0].nbytes, offset=2 * e) for _ in range(ndst)]  # one residue mod 16
    bufs = snac.snac_coll_desc()
    bufs.ndst = ndst
    for k, b in enumerate(sb):
        bufs.src[k] = b.ptr
    for k, b in enumerate(db):
        bufs.dst[k] = b.ptr
    launch(dev.devtest_reduce_slices(ctypes.byref(bufs), nsrc, per, blocks, int(dtype == "bf16"), None))
    sync()
    want = oracle.reduce_n(srcs, dtype)
    for k, b in enumerate(db):
        assert b.guards_ok()
        assert_same(b.download(np_dtype(dtype)), want, dtype, f"snac::reduce N={nsrc} dst[{k}]")


# ------------------------------------------------- device-side collectives
def _case(coll, n, dtype, m, misalign, seed):
    """Inputs, destination buffers, describe arguments and the oracle's
    outputs for one collective."""
    e = np.dtype(np_dtype(dtype)).itemsize
    off = e if misalign else 0
    counts = None
    if coll in (snac.SNAC_COLL_ALL_GATHER_V, snac.SNAC_COLL_REDUCE_SCATTER_V):
        counts = [int(c) for c in wl.v_counts(n, m, 1, cfg=wl.CFG_TEST, seed=seed)[0]]
    if coll == snac.SNAC_COLL_ALL_TO_ALL_V:
        counts = wl.v_counts(n, m, n, cfg=wl.CFG_TEST, seed=seed)
    if coll == snac.SNAC_COLL_ALL_GATHER_V:
        srcs = [gen(1, counts[k], dtype, seed + k)[0] for k in range(n)]
    else:
        srcs = gen(n, m, dtype, seed)
    if coll == snac.SNAC_COLL_ALL_REDUCE:
        want = oracle.all_reduce(srcs, dtype)
    elif coll == snac.SNAC_COLL_REDUCE_SCATTER:
        want = oracle.reduce_scatter(srcs, dtype)
    elif coll == snac.SNAC_COLL_ALL_GATHER:
        want = oracle.all_gather(srcs)
    elif coll == snac.SNAC_COLL_ALL_TO_ALL:
        want = oracle.all_to_all(srcs)
    elif coll == snac.SNAC_COLL_ALL_GATHER_V:
        want = oracle.all_gather_v(srcs, counts)
    elif coll == snac.SNAC_COLL_REDUCE_SCATTER_V:
        want = oracle.reduce_scatter_v(srcs, counts, dtype)
    else:
        want = oracle.all_to_all_v(srcs, counts)
    sb = [DevBuf(s.nbytes, offset=off * (k % 3), data=s) for k, s in enumerate(srcs)]
    db = [DevBuf(np.asarray(w).nbytes, offset=off) for w in want]
    flat = None if counts is None else np.asarray(counts).reshape(-1).tolist()
    return srcs, sb, db, want, srcs[0].nbytes, flat


COLLS = [
    (snac.SNAC_COLL_ALL_REDUCE, "bf16"),
    (snac.SNAC_COLL_ALL_REDUCE, "f32"),
    (snac.SNAC_COLL_REDUCE_SCATTER, "bf16"),
    (snac.SNAC_COLL_ALL_GATHER, "u32"),
    (snac.SNAC_COLL_ALL_TO_ALL, "byte"),
    (snac.SNAC_COLL_ALL_GATHER_V, "bf16"),
    (snac.SNAC_COLL_REDUCE_SCATTER_V, "f32"),
    (snac.SNAC_COLL_ALL_TO_ALL_V, "u32"),
]


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("coll,dtype", COLLS)
def test_device_collective(dev, ctx8, coll, dtype, misalign):
    n = 8
    m = 8 * 12_289  # divisible by N for RS / A2A; several 16 KiB tiles per job
    srcs, sb, db, want, nbytes, counts = _case(coll, n, dtype, m, misalign, seed=coll * 10 + int(misalign))
    desc = snac.snac_describe(ctx8, coll, [b.ptr for b in sb], [b.ptr for b in db], nbytes, counts, dtype)
    if misalign:
        assert not desc.flags & snac.SNAC_DESC_ALIGNED
    dctx = snac.snac_get_device_context(ctx8)
    blocks, coll_blocks, extra = 48, 32, 16
    ok = ok_buffer(blocks + extra)
    launch(dev.devtest_collective(ctypes.byref(desc), ctypes.byref(dctx), int(dtype == "bf16"), n, blocks,
                                  coll_blocks, extra, 0, ok.data_ptr(), None))
    sync()
    snac.snac_check(ctx8)
    assert ok[:blocks].cpu().numpy().tolist() == [1] * blocks
    assert ok[blocks:].cpu().numpy().tolist() == [0] * extra
    for r, (b, w) in enumerate(zip(db, want)):
        assert b.guards_ok(), f"canary around dst[{r}]"
        assert_same(b.download(np_dtype(dtype)), np.asarray(w), dtype, f"device collective {coll} dst[{r}]")


@pytest.mark.parametrize("blocks", [37, 1500])
@pytest.mark.parametrize("coll,dtype", COLLS)
def test_device_collective_without_barrier(dev, ctx8, coll, dtype, blocks):
    """SYNC = false: no closing grid barrier, so any grid size works (1500
    workgroups exceed what fits at once); the output is complete after the
    kernel."""
    n = 8
    m = 8 * 12_289
    srcs, sb, db, want, nbytes, counts = _case(coll, n, dtype, m, blocks == 37, seed=coll * 10 + 7)
    desc = snac.snac_describe(ctx8, coll, [b.ptr for b in sb], [b.ptr for b in db], nbytes, counts, dtype)
    dctx = snac.snac_get_device_context(ctx8)
    ok = ok_buffer(blocks)
    launch(dev.devtest_collective_nosync(ctypes.byref(desc), ctypes.byref(dctx), int(dtype == "bf16"), n, blocks,
                                         ok.data_ptr(), None))
    sync()
    snac.snac_check(ctx8)
    assert int(ok.sum().item()) == blocks
    for r, (b, w) in enumerate(zip(db, want)):
        assert b.guards_ok(), f"canary around dst[{r}]"
        assert_same(b.download(np_dtype(dtype)), np.asarray(w), dtype, f"no-barrier collective {coll} dst[{r}]")


def test_device_collective_repeats_and_one_block(dev, ctx8):
    """The barrier's generation carries across calls; one workgroup alone
    also completes a collective."""
    n, m = 8, 40_000
    srcs, sb, db, want, nbytes, _ = _case(snac.SNAC_COLL_ALL_REDUCE, n, "bf16", m, False, seed=3)
    desc = snac.snac_describe(ctx8, snac.SNAC_COLL_ALL_REDUCE, [b.ptr for b in sb], [b.ptr for b in db], nbytes,
                              None, "bf16")
    dctx = snac.snac_get_device_context(ctx8)
    for blocks, coll_blocks in [(1, 1), (200, 200), (64, 1), (7, 5)]:
        for b in db:
            b.t.fill_(0xA5)
        ok = ok_buffer(blocks)
        launch(dev.devtest_collective(ctypes.byref(desc), ctypes.byref(dctx), 1, n, blocks, coll_blocks, 0, 0,
                                      ok.data_ptr(), None))
        sync()
        snac.snac_check(ctx8)
        assert int(ok.sum().item()) == blocks
        for r, (b, w) in enumerate(zip(db, want)):
            assert_same(b.download(np.uint16), w, "bf16", f"blocks={blocks} dst[{r}]")


def test_device_collective_mismatch_latches_arg(dev, ctx8):
    n, m = 8, 4096
    srcs, sb, db, want, nbytes, _ = _case(snac.SNAC_COLL_ALL_REDUCE, n, "f32", m, False, seed=9)
    desc = snac.snac_describe(ctx8, snac.SNAC_COLL_ALL_REDUCE, [b.ptr for b in sb], [b.ptr for b in db], nbytes,
                              None, "f32")
    dctx = snac.snac_get_device_context(ctx8)
    ok = ok_buffer(16)
    # the kernel is instantiated for N = 3 sources, the descriptor has 8
    launch(dev.devtest_collective(ctypes.byref(desc), ctypes.byref(dctx), 0, 3, 16, 16, 0, 0, ok.data_ptr(), None))
    sync()
    assert int(ok.sum().item()) == 0
    for b in db:
        assert np.all(b.download() == 0xA5), "nothing may be written on a mismatch"
    with pytest.raises(snac.SnacError) as e:
        snac.snac_check(ctx8)
    assert e.value.status == snac.SNAC_E_ARG
    # re-armed: the same descriptor with matching template arguments works
    ok = ok_buffer(16)
    launch(dev.devtest_collective(ctypes.byref(desc), ctypes.byref(dctx), 0, 8, 16, 16, 0, 0, ok.data_ptr(), None))
    sync()
    snac.snac_check(ctx8)
    for r, (b, w) in enumerate(zip(db, want)):
        assert_same(b.download(np.float32), w, "f32", f"after re-arm dst[{r}]")


def test_device_collective_null_workspace_latches_arg(dev, ctx8):
    """A call without an LDS workspace moves nothing and latches SNAC_E_ARG;
    every participant returns false without waiting."""
    n, m = 8, 4096
    srcs, sb, db, want, nbytes, _ = _case(snac.SNAC_COLL_ALL_REDUCE, n, "f32", m, False, seed=10)
    desc = snac.snac_describe(ctx8, snac.SNAC_COLL_ALL_REDUCE, [b.ptr for b in sb], [b.ptr for b in db], nbytes,
                              None, "f32")
    dctx = snac.snac_get_device_context(ctx8)
    ok = ok_buffer(16)
    launch(dev.devtest_collective(ctypes.byref(desc), ctypes.byref(dctx), 0, 8, 16, 16, 0, 1, ok.data_ptr(), None))
    sync()
    assert int(ok.sum().item()) == 0
    for b in db:
        assert np.all(b.download() == 0xA5), "nothing may be written without a workspace"
    with pytest.raises(snac.SnacError) as e:
        snac.snac_check(ctx8)
    assert e.value.status == snac.SNAC_E_ARG


def test_atom_launch_contract(dev):
    """The published launch contract: THREADS threads per workgroup, and the
    dynamic LDS that holds everything collective() keeps in LDS (256 jobs of
    the table, the scan, the barrier word) -- the test kernels that call it
    declare no static LDS of their own, and copy() needs none."""
    import ctypes as ct

    out = (ct.c_uint32 * 5)()
    launch(dev.devtest_atom_contract(out))
    threads, pipeline, copy_lds, reduce_lds, coll = list(out)
    assert threads == 256
    assert copy_lds == 0 and reduce_lds == 0
    assert pipeline == coll
    assert 256 * 40 + 256 * 4 + 4 <= coll <= 64 * 1024 and coll % 128 == 0
    for which in range(4):
        v = ct.c_uint32(0xFFFFFFFF)
        launch(dev.devtest_static_lds(which, ct.byref(v)))
        assert v.value == 0, f"test kernel {which} declares {v.value} bytes of static LDS"


# --------------------------------- compute + in-kernel AllReduce + compute
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [3, 8])
def test_fused_scale_allreduce(dev, dtype, n):
    import torch

    e = 2 if dtype == "bf16" else 4
    count = 100_003
    if dtype == "bf16":
        xs = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r) for r in range(n)]
    else:
        xs = [wl.normal_f32(count, wl.CFG_PIPELINE_N8, r) for r in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        xb = [DevBuf(count * e, data=x) for x in xs]
        tmp = [DevBuf(count * e) for _ in range(n)]
        out = [DevBuf(count * e) for _ in range(n)]
        check = DevBuf(count * e)
        desc = snac.snac_describe(ctx, snac.SNAC_COLL_ALL_REDUCE, [b.ptr for b in tmp], [b.ptr for b in out],
                                  count * e, None, dtype)
        xsd = snac.snac_coll_desc()
        for r, b in enumerate(xb):
            xsd.src[r] = b.ptr
        dctx = snac.snac_get_device_context(ctx)
        want = oracle.pipeline_scale_reduce(xs, dtype)
        for rep in range(2):
            blocks = 128 if rep == 0 else 33
            ok = ok_buffer(blocks)
            check.t.fill_(0xA5)
            launch(dev.devtest_fused_scale_allreduce(ctypes.byref(desc), ctypes.byref(dctx), ctypes.byref(xsd), count,
                                                     check.ptr, blocks, ok.data_ptr(), None))
            torch.cuda.synchronize()
            snac.snac_check(ctx)
            assert int(ok.sum().item()) == blocks
            for r, b in enumerate(out):
                assert b.guards_ok()
                assert_same(b.download(np_dtype(dtype)), want, dtype, f"fused N={n} out[{r}] rep {rep}")
            assert check.guards_ok()
            assert_same(check.download(np_dtype(dtype)), want, dtype, f"fused N={n} read-back rep {rep}")
    finally:
        snac.snac_finalize(ctx)


# ------------------------------------------ SNAC primitives used by hand
@pytest.mark.parametrize("n,S", [(2, 2), (8, 2), (8, 3)])
def test_stage_notify_consume_by_hand(dev, n, S):
    """n producer workgroups stage blocks and notify; one consumer consumes
    every rank's flag, reduces the staged blocks and frees the slot; slots
    are reused (R > S) and the sequence numbers keep rising across calls."""
    import torch

    R, B = 7, 5000
    xs = [wl.uniform_f32(R * B, wl.CFG_TEST, r, seed=n * 10 + S) for r in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        xb = [DevBuf(x.nbytes, data=x) for x in xs]
        xsd = snac.snac_coll_desc()
        for r, b in enumerate(xb):
            xsd.src[r] = b.ptr
        stage = torch.zeros(n * S * B, dtype=torch.float32, device="cuda")
        dctx = snac.snac_get_device_context(ctx)
        want = np.stack([oracle.reduce_n([x[r * B:(r + 1) * B] for x in xs], "f32") for r in range(R)])
        base = 0
        for call in range(2):
            out = torch.full((R * B,), -1.0, dtype=torch.float32, device="cuda")
            ok = ok_buffer(n + 1)
            launch(dev.devtest_flags(ctypes.byref(dctx), ctypes.byref(xsd), stage.data_ptr(), out.data_ptr(), n, S, R,
                                     B, base, ok.data_ptr(), None))
            torch.cuda.synchronize()
            snac.snac_check(ctx)
            assert int(ok.sum().item()) == n + 1
            assert_same(out.cpu().numpy().reshape(R, B), want, "f32", f"n={n} S={S} call {call}")
            base += R
    finally:
        snac.snac_finalize(ctx)


@pytest.mark.parametrize("K", [1, 63, 64, 65, 130, 1000])
def test_consume_many_flags(dev, K):
    """One consumer waits on K flags at once: one lane per flag, in groups
    of 64.  Each producer's value must be visible after the consume."""
    import torch

    ctx = snac.snac_init(2, 0)
    try:
        dctx = snac.snac_get_device_context(ctx)
        vals = torch.zeros(K, dtype=torch.int32, device="cuda")
        total = torch.zeros(1, dtype=torch.int64, device="cuda")
        for call in range(2):  # flags are never reset: the target rises
            vals.zero_()
            ok = ok_buffer(K + 1)
            launch(dev.devtest_many_flags(ctypes.byref(dctx), vals.data_ptr(), K, call + 1, total.data_ptr(),
                                          ok.data_ptr(), None))
            torch.cuda.synchronize()
            snac.snac_check(ctx)
            assert int(ok.sum().item()) == K + 1
            assert int(total.item()) == K * (K + 1) // 2
    finally:
        snac.snac_finalize(ctx)
