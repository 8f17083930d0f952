"""Whole-output parity of the copy kernels in their big-message shapes.

One-to-one copies that move at least 1 GiB (bytes read plus bytes written)
run single-wave workgroups on grid-stride 4 KiB tiles, five per CU, when
the call has no context (snac_copy) or its tile schedule is grid-stride
only; a collective call with a context instead hands 16 KiB tiles out in
order from its tile counters.  Copies whose source sits at a byte offset
from the destination's dword grid keep 256-thread workgroups on 16 KiB
tiles, whose full tiles take the next lane's bytes through DPP shifts.
Sampled checks at the benchmark sizes could miss a single lost tile, so
here every output byte is compared with the oracle, aligned and
misaligned, with ragged tails, under both schedules, and the canary bytes
around every destination must be untouched."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from gpu_helpers import DevBuf, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MiB = 1 << 20


def sync():
    import torch

    torch.cuda.synchronize()


def rand_bytes(n: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, 256, size=n, dtype=np.uint8)


@pytest.mark.parametrize("src_off,dst_off,nbytes", [
    (0, 0, 512 * MiB + 3 * 4096 + 5 * 16),  # aligned, partial last tile
    (4, 12, 512 * MiB + 4093),              # 4-byte aligned, different offsets, odd tail
    (1, 0, 513 * MiB + 7),                  # byte-misaligned source (16 KiB tiles, DPP shifts)
    (7, 2, 512 * MiB + 9),                  # source 5 bytes off the destination's dword grid
])
def test_copy_moving_a_gib_or_more(src_off, dst_off, nbytes):
    assert 2 * nbytes >= 1 << 30
    data = rand_bytes(nbytes, seed=src_off * 16 + dst_off)
    sb = DevBuf(nbytes, offset=src_off, data=data)
    db = DevBuf(nbytes, offset=dst_off)
    snac.snac_copy(db.ptr, sb.ptr, nbytes)
    sync()
    got = db.download()
    want = oracle.copy(data)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {int(bad[0])}"
    assert db.guards_ok()


@pytest.fixture(params=[0, 1], ids=["counters", "grid-stride"])
def schedule(request):
    t0 = snac.snac_get_tuning()
    snac.snac_set_tuning(tile_schedule=request.param)
    yield request.param
    snac.snac_set_tuning(**t0)


@pytest.mark.parametrize("n,chunk_bytes,offset", [
    (4, 64 * MiB + 4096, 0),  # every chunk 16-byte aligned
    (4, 64 * MiB + 12, 0),    # chunk starts 4-byte aligned only
    (2, 256 * MiB + 8, 4),    # two ranks, buffers 4 bytes off
])
def test_all_to_all_moving_a_gib_or_more(schedule, n, chunk_bytes, offset):
    per_rank = n * chunk_bytes
    assert 2 * n * per_rank >= 1 << 30
    e = per_rank // 4
    host = [rand_bytes(per_rank, seed=100 + r).view(np.uint32) for r in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        sb = [DevBuf(per_rank, offset=offset, data=h) for h in host]
        db = [DevBuf(per_rank, offset=offset) for _ in range(n)]
        snac.snac_all_to_all(ctx, [b.ptr for b in sb], [b.ptr for b in db], per_rank, "u32")
        sync()
        snac.snac_check(ctx)
    finally:
        snac.snac_finalize(ctx)
    want = oracle.all_to_all(host)
    for d in range(n):
        got = db[d].download(np.uint32)
        assert got.size == e
        bad = np.flatnonzero(got != want[d])
        assert bad.size == 0, f"dst[{d}]: {bad.size} words differ, first at {int(bad[0])}"
        assert db[d].guards_ok()


def test_byte_all_to_all_moving_a_gib_or_more(schedule):
    # chunks of 64 MiB + 3 bytes: every job but the first reads at a byte
    # offset from its destination's dword grid (16 KiB tiles, DPP shifts)
    n, chunk_bytes = 4, 64 * MiB + 3
    per_rank = n * chunk_bytes
    assert 2 * n * per_rank >= 1 << 30
    host = [rand_bytes(per_rank, seed=200 + r) for r in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        sb = [DevBuf(per_rank, offset=1, data=h) for h in host]
        db = [DevBuf(per_rank, offset=0) for _ in range(n)]
        snac.snac_all_to_all(ctx, [b.ptr for b in sb], [b.ptr for b in db], per_rank, "byte")
        sync()
        snac.snac_check(ctx)
    finally:
        snac.snac_finalize(ctx)
    want = oracle.all_to_all(host)
    for d in range(n):
        got = db[d].download()
        bad = np.flatnonzero(got != want[d])
        assert bad.size == 0, f"dst[{d}]: {bad.size} bytes differ, first at {int(bad[0])}"
        assert db[d].guards_ok()
