"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, bit-exact, on seeded inputs at sizes that span several
tiles and end in a ragged tail.  Every destination is surrounded by canary
bytes that must survive the call."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import DevBuf, assert_same, gpu_available, np_dtype

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sync():
    import torch

    torch.cuda.synchronize()


def gen(n: int, m: int, dtype: str, seed: int = 1):
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "u32":
        return [wl.raw_u32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


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


def run_and_check(dsts, wants, dtype, what):
    sync()
    for r, (b, w) in enumerate(zip(dsts, wants)):
        assert b.guards_ok(), f"{what}: canary overwritten around dst[{r}]"
        assert_same(b.download(np_dtype(dtype)), np.asarray(w), dtype, f"{what} dst[{r}]")


# ------------------------------------------------------------ worked example
def test_worked_example_allreduce(ctxs):
    with open(os.path.join(GOLDEN, "nki_allreduce_worked_example.json")) as f:
        g = json.load(f)
    srcs = [np.asarray(x, dtype=np.float32).reshape(-1) for x in g["inputs"]]
    want = [np.asarray(x, dtype=np.float32).reshape(-1) for x in g["expected"]]
    sb = [DevBuf(s.nbytes, data=s) for s in srcs]
    db = [DevBuf(s.nbytes) for s in srcs]
    snac.snac_all_reduce(ctxs(2), [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, "f32")
    run_and_check(db, want, "f32", "worked example")


def test_allreduce_f32_n2_1kib(ctxs):
    srcs = [wl.uniform_f32(256, wl.CFG_AR_F32_N2, r) for r in range(2)]
    sb = [DevBuf(1024, data=s) for s in srcs]
    db = [DevBuf(1024) for _ in srcs]
    snac.snac_all_reduce(ctxs(2), [b.ptr for b in sb], [b.ptr for b in db], 1024, "f32")
    run_and_check(db, oracle.all_reduce(srcs, "f32"), "f32", "AR f32 N=2 1KiB")


# ------------------------------------------------------------------ reduce
AR_SIZES = [1, 7, 8, 1000, 4096, 3 * 8192 + 24, 100_003]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 16])
def test_allreduce(ctxs, n, dtype):
    for m in AR_SIZES:
        srcs = gen(n, m, dtype, seed=m)
        nb = srcs[0].nbytes
        sb = [DevBuf(nb, data=s) for s in srcs]
        db = [DevBuf(nb) for _ in srcs]
        snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], nb, dtype)
        run_and_check(db, oracle.all_reduce(srcs, dtype), dtype, f"AR N={n} {dtype} m={m}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_allreduce_misaligned_and_inplace(ctxs, dtype):
    n, m = 8, 20_011
    e = 2 if dtype == "bf16" else 4
    srcs = gen(n, m, dtype, seed=5)
    want = oracle.all_reduce(srcs, dtype)
    for so, do in [(e, 0), (0, e), (3 * e, 5 * e), (4, 12), (6 * e, 6 * e)]:
        sb = [DevBuf(srcs[0].nbytes, offset=so + (r * e) % 16, data=s) for r, s in enumerate(srcs)]
        db = [DevBuf(srcs[0].nbytes, offset=do) for _ in srcs]
        snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, dtype)
        run_and_check(db, want, dtype, f"AR misaligned src+{so} dst+{do}")
    # destinations with different residues modulo 16 (split multicast)
    sb = [DevBuf(srcs[0].nbytes, data=s) for s in srcs]
    db = [DevBuf(srcs[0].nbytes, offset=(r * e) % 16) for r in range(n)]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], srcs[0].nbytes, dtype)
    run_and_check(db, want, dtype, "AR mixed dst residues")
    # in place
    sb = [DevBuf(srcs[0].nbytes, data=s) for s in srcs]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in sb], srcs[0].nbytes, dtype)
    run_and_check(sb, want, dtype, "AR in place")


def test_bf16_rounding_ties(ctxs):
    # pairs whose binary32 sum sits exactly halfway between bf16 values
    a = np.array([0x3F80, 0x3F81, 0x3F80, 0xBF80, 0x4380, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    b = np.array([0x3B80, 0x3B80, 0x3BC0, 0xBB80, 0x3F80, 0x0001, 0x7B00, 0x8000], dtype=np.uint16)
    a = np.tile(a, 64)
    b = np.tile(b, 64)
    sb = [DevBuf(a.nbytes, data=a), DevBuf(b.nbytes, data=b)]
    db = [DevBuf(a.nbytes) for _ in range(2)]
    snac.snac_all_reduce(ctxs(2), [x.ptr for x in sb], [x.ptr for x in db], a.nbytes, "bf16")
    run_and_check(db, oracle.all_reduce([a, b], "bf16"), "bf16", "bf16 ties")
    # all -0.0 keeps the sign (accumulator starts from rank 0's value)
    z = np.full(64, 0x8000, dtype=np.uint16)
    sb = [DevBuf(z.nbytes, data=z) for _ in range(3)]
    db = [DevBuf(z.nbytes) for _ in range(3)]
    snac.snac_all_reduce(ctxs(3), [x.ptr for x in sb], [x.ptr for x in db], z.nbytes, "bf16")
    run_and_check(db, oracle.all_reduce([z, z, z], "bf16"), "bf16", "-0")


def test_rank_order_matters(ctxs):
    # (2^24 + 1) - 2^24 = 0 in rank order; any other order gives 1
    vals = [np.full(1024, v, dtype=np.float32) for v in (2.0 ** 24, 1.0, -(2.0 ** 24))]
    sb = [DevBuf(v.nbytes, data=v) for v in vals]
    db = [DevBuf(v.nbytes) for v in vals]
    snac.snac_all_reduce(ctxs(3), [x.ptr for x in sb], [x.ptr for x in db], vals[0].nbytes, "f32")
    run_and_check(db, [np.zeros(1024, dtype=np.float32)] * 3, "f32", "rank order")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reduce_n_atom(dtype):
    m = 33_333
    for nsrc, ndst in [(1, 1), (3, 1), (8, 2), (16, 16), (5, 3)]:
        srcs = gen(nsrc, m, dtype, seed=nsrc * 10 + ndst)
        sb = [DevBuf(srcs[0].nbytes, data=s) for s in srcs]
        db = [DevBuf(srcs[0].nbytes, offset=(2 * k) if dtype == "bf16" else 0) for k in range(ndst)]
        snac.snac_reduce_n([b.ptr for b in db], [b.ptr for b in sb], m, dtype)
        want = oracle.reduce_n(srcs, dtype)
        run_and_check(db, [want] * ndst, dtype, f"reduceN {nsrc}->{ndst}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
def test_reduce_scatter(ctxs, n, dtype):
    for mc in [1, 5, 4096, 12_345]:
        srcs = gen(n, n * mc, dtype, seed=mc)
        nb = srcs[0].nbytes
        sb = [DevBuf(nb, data=s) for s in srcs]
        db = [DevBuf(nb // n) for _ in srcs]
        snac.snac_reduce_scatter(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], nb, dtype)
        run_and_check(db, oracle.reduce_scatter(srcs, dtype), dtype, f"RS N={n} mc={mc}")


# ------------------------------------------------------------------- copy
@pytest.mark.parametrize("dtype", ["byte", "u32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
def test_all_gather(ctxs, n, dtype):
    for m in [1, 3, 4096, 9_999]:
        srcs = gen(n, m, dtype, seed=m + n)
        nb = srcs[0].nbytes
        sb = [DevBuf(nb, data=s) for s in srcs]
        db = [DevBuf(n * nb) for _ in srcs]
        snac.snac_all_gather(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], nb, dtype)
        run_and_check(db, oracle.all_gather(srcs), dtype, f"AG N={n} {dtype} m={m}")


@pytest.mark.parametrize("dtype", ["byte", "u32", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
def test_all_to_all(ctxs, n, dtype):
    for mc in [1, 7, 4096, 5_001]:
        srcs = gen(n, n * mc, dtype, seed=mc)
        nb = srcs[0].nbytes
        sb = [DevBuf(nb, data=s) for s in srcs]
        db = [DevBuf(nb) for _ in srcs]
        snac.snac_all_to_all(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], nb, dtype)
        run_and_check(db, oracle.all_to_all(srcs), dtype, f"A2A N={n} mc={mc}")


@pytest.mark.parametrize("nbytes", [0, 1, 15, 16, 17, 255, 4096, 65_536 + 3, 1_000_001])
def test_copy_any_alignment(nbytes):
    data = wl.raw_bytes(nbytes, wl.CFG_TEST, 0, seed=nbytes)
    for so, do in [(0, 0), (1, 0), (0, 1), (3, 2), (2, 3), (4, 8), (7, 13), (12, 4), (15, 1)]:
        s = DevBuf(nbytes, offset=so, data=data)
        d = DevBuf(nbytes, offset=do)
        snac.snac_copy(d.ptr, s.ptr, nbytes)
        run_and_check([d], [oracle.copy(data)], "byte", f"copy {nbytes} src+{so} dst+{do}")


# -------------------------------------------------------------- V variants
def _v_counts(n, total, rows, seed):
    return wl.v_counts(n, total, rows, cfg=wl.CFG_TEST + seed)


@pytest.mark.parametrize("dtype", ["u32", "f32", "bf16", "byte"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_all_to_all_v(ctxs, n, dtype):
    for total, seed in [(10_000, 1), (100_003, 2), (7, 3)]:
        c = _v_counts(n, total, n, seed)
        srcs = gen(n, total, dtype, seed=seed)
        sb = [DevBuf(s.nbytes, data=s) for s in srcs]
        want = oracle.all_to_all_v(srcs, c)
        db = [DevBuf(w.nbytes) for w in want]
        snac.snac_all_to_all_v(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], c.reshape(-1).tolist(), dtype)
        run_and_check(db, want, dtype, f"A2AV N={n} total={total}")


@pytest.mark.parametrize("dtype", ["u32", "bf16", "byte"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_all_gather_v(ctxs, n, dtype):
    for total, seed in [(10_000, 4), (99_999, 5), (5, 6)]:
        c = _v_counts(n, total, 1, seed)[0]
        srcs = [gen(1, max(1, int(c[k])), dtype, seed=seed + k)[0][: int(c[k])] for k in range(n)]
        sb = [DevBuf(s.nbytes, data=s) for s in srcs]
        want = oracle.all_gather_v(srcs, list(c))
        db = [DevBuf(w.nbytes) for w in want]
        snac.snac_all_gather_v(ctxs(n), [b.ptr if b.nbytes else b.ptr for b in sb], [b.ptr for b in db], c.tolist(), dtype)
        run_and_check(db, want, dtype, f"AGV N={n} total={total}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_reduce_scatter_v(ctxs, n, dtype):
    for total, seed in [(10_000, 7), (100_001, 8), (9, 9)]:
        c = _v_counts(n, total, 1, seed)[0]
        srcs = gen(n, total, dtype, seed=seed)
        sb = [DevBuf(s.nbytes, data=s) for s in srcs]
        want = oracle.reduce_scatter_v(srcs, list(c), dtype)
        db = [DevBuf(w.nbytes) for w in want]
        snac.snac_reduce_scatter_v(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], c.tolist(), dtype)
        run_and_check(db, want, dtype, f"RSV N={n} total={total}")


def test_v_equal_counts_match_fixed(ctxs):
    n, mc = 8, 3000
    srcs = gen(n, n * mc, "f32", seed=77)
    nb = srcs[0].nbytes
    sb = [DevBuf(nb, data=s) for s in srcs]
    d1 = [DevBuf(nb) for _ in srcs]
    d2 = [DevBuf(nb) for _ in srcs]
    snac.snac_all_to_all(ctxs(n), [b.ptr for b in sb], [b.ptr for b in d1], nb, "f32")
    snac.snac_all_to_all_v(ctxs(n), [b.ptr for b in sb], [b.ptr for b in d2], [mc] * (n * n), "f32")
    sync()
    for a, b in zip(d1, d2):
        assert np.array_equal(a.download(), b.download())


# -------------------------------------------------------- SNAC pipeline
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
def test_pipeline(n, dtype):
    ctx = snac.snac_init(n, 4 * 65536)  # 4 slots: the ring wraps many times
    try:
        for count in [1, 5, 32768 + 3, 300_001]:
            xs = gen(n, count, dtype, seed=count)
            xb = [DevBuf(x.nbytes, data=x) for x in xs]
            ob = DevBuf(xs[0].nbytes)
            snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in xb], ob.ptr, count, dtype)
            snac.snac_check(ctx)
            run_and_check([ob], [oracle.pipeline_scale_reduce(xs, dtype)], dtype, f"pipeline N={n} count={count}")
    finally:
        snac.snac_finalize(ctx)


@pytest.mark.parametrize("tile,lookahead,wgs", [(4096, 1, 1), (8192, 0, 1), (12288, 2, 1), (16384, 3, 2), (65536, 0, 4),
                                                (262144, 7, 1)])
def test_pipeline_tunings(tile, lookahead, wgs):
    n, dtype = 5, "bf16"
    t0 = snac.snac_get_tuning()
    try:
        snac.snac_set_tuning(pipeline_tile_bytes=tile, pipeline_lookahead=lookahead, wgs_per_cu=wgs)
        ctx = snac.snac_init(n, 16 * tile)
        try:
            for count in [tile // 2 * 3 + 7, 40 * tile // 2 + 1]:
                xs = gen(n, count, dtype, seed=count + tile)
                xb = [DevBuf(x.nbytes, data=x) for x in xs]
                ob = DevBuf(xs[0].nbytes)
                snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in xb], ob.ptr, count, dtype)
                snac.snac_check(ctx)
                run_and_check([ob], [oracle.pipeline_scale_reduce(xs, dtype)], dtype, f"pipeline tile={tile} count={count}")
        finally:
            snac.snac_finalize(ctx)
    finally:
        snac.snac_set_tuning(**t0)


KiB, MiB = 1 << 10, 1 << 20


@pytest.mark.parametrize("n,ring,count,dtype", [
    (8, 8 * MiB, (1 << 20) + 3, "bf16"),     # fits the ring: tiles split to 64 KiB, 33 tiles, compacted slots
    (8, 4 * MiB, 5 * (1 << 20) + 3, "bf16"),  # 10 MiB through a 4 MiB ring: slots merged, several passes
    (4, 64 * MiB, 47107, "bf16"),              # 5 units + 3 pieces + 6 bytes in a large ring
    (16, 16 * MiB, (2 << 20) + 3, "bf16"),     # 16 ranks: 4 KiB units
    (3, 2 * MiB, 1_000_003, "f32"),            # 4 MB through a 2 MiB ring
    (2, 64 * MiB, 8 * (1 << 20) + 1, "f32"),   # N=2: 132 tiles of 256 KiB, one element past the last unit
])
def test_pipeline_layouts(n, ring, count, dtype):
    """Default tiles across ring sizes, rank counts and short last units: the
    call re-cuts the ring (merged or split slots, compacted when the message
    fits) and tiles own interleaved units of the message."""
    ctx = snac.snac_init(n, ring)
    try:
        xs = gen(n, count, dtype, seed=count % 1000 + n)
        xb = [DevBuf(x.nbytes, data=x) for x in xs]
        ob = DevBuf(xs[0].nbytes)
        snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in xb], ob.ptr, count, dtype)
        snac.snac_check(ctx)
        run_and_check([ob], [oracle.pipeline_scale_reduce(xs, dtype)], dtype, f"pipeline N={n} ring={ring} count={count}")
    finally:
        snac.snac_finalize(ctx)


def test_pipeline_alternating_inputs():
    """Consecutive calls with different inputs: a consumer that read stale
    staged data from an earlier call would produce the other output."""
    n, count, dtype = 8, 150_001, "bf16"
    ctx = snac.snac_init(n, 16 * 32768)
    try:
        sets = [gen(n, count, dtype, seed=s) for s in (41, 42)]
        want = [oracle.pipeline_scale_reduce(xs, dtype) for xs in sets]
        bufs = [[DevBuf(x.nbytes, data=x) for x in xs] for xs in sets]
        outs = [DevBuf(sets[0][0].nbytes) for _ in range(12)]
        for i, ob in enumerate(outs):
            snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in bufs[i % 2]], ob.ptr, count, dtype)
        snac.snac_check(ctx)
        run_and_check(outs, [want[i % 2] for i in range(len(outs))], dtype, "pipeline alternating inputs")
    finally:
        snac.snac_finalize(ctx)


def test_pipeline_alternating_queue_counts():
    """Calls of one tile (one queue, which finishes without the global done
    count) alternating with calls over several queues, back to back on one
    context: every output checked, so a done count or epoch left wrong by
    either completion path would show as a timeout or stale data."""
    n, dtype = 8, "bf16"
    ctx = snac.snac_init(n, 8 * MiB)
    try:
        counts = [512, 2 * MiB + 7, 3, 4 * MiB // 2, 1024 + 1, 1 * MiB + 5] * 3
        data = {c: gen(n, c, dtype, seed=c % 997) for c in set(counts)}
        bufs = {c: [DevBuf(x.nbytes, data=x) for x in xs] for c, xs in data.items()}
        outs = [DevBuf(data[c][0].nbytes) for c in counts]
        for c, ob in zip(counts, outs):
            snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in bufs[c]], ob.ptr, c, dtype)
        snac.snac_check(ctx)
        want = {c: oracle.pipeline_scale_reduce(xs, dtype) for c, xs in data.items()}
        run_and_check(outs, [want[c] for c in counts], dtype, "pipeline alternating queue counts")
    finally:
        snac.snac_finalize(ctx)


def test_pipeline_back_to_back():
    n, count, dtype = 8, 200_000, "bf16"
    ctx = snac.snac_init(n, 8 * 65536)
    try:
        xs = gen(n, count, dtype, seed=3)
        xb = [DevBuf(x.nbytes, data=x) for x in xs]
        outs = [DevBuf(xs[0].nbytes) for _ in range(50)]
        for ob in outs:
            snac.snac_pipeline_scale_reduce(ctx, [b.ptr for b in xb], ob.ptr, count, dtype)
        snac.snac_check(ctx)
        want = oracle.pipeline_scale_reduce(xs, dtype)
        run_and_check(outs, [want] * len(outs), dtype, "pipeline back to back")
    finally:
        snac.snac_finalize(ctx)


# --------------------------------------------------------- determinism
def test_repeat_runs_bit_identical(ctxs):
    n, m = 8, 1 << 20
    srcs = gen(n, m, "bf16", seed=99)
    sb = [DevBuf(srcs[0].nbytes, data=s) for s in srcs]
    d1 = [DevBuf(srcs[0].nbytes) for _ in srcs]
    d2 = [DevBuf(srcs[0].nbytes) for _ in srcs]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in d1], srcs[0].nbytes, "bf16")
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in d2], srcs[0].nbytes, "bf16")
    sync()
    for a, b in zip(d1, d2):
        assert np.array_equal(a.download(), b.download())


# -------------------------------------------- 16 KiB-tile (large-message) paths
# Messages with fewer 16 KiB tiles than the GPU has CUs run the small-tile
# kernels, so the cases above mostly exercise those; these sizes (over 4 MiB
# per rank) keep the 16 KiB-tile kernels, misaligned (generic) and ragged.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_tiles_misaligned_allreduce_and_rs(ctxs, dtype):
    n = 8
    e = 2 if dtype == "bf16" else 4
    m = 8 * (600_000 + 13)  # > 4 MiB per rank, divisible by N, ragged
    srcs = gen(n, m, dtype, seed=41)
    nb = srcs[0].nbytes
    sb = [DevBuf(nb, offset=e * (k % 4), data=s) for k, s in enumerate(srcs)]
    db = [DevBuf(nb, offset=e) for _ in srcs]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], nb, dtype)
    run_and_check(db, oracle.all_reduce(srcs, dtype), dtype, f"AR large misaligned {dtype}")
    rb = [DevBuf(nb // n, offset=3 * e) for _ in srcs]
    snac.snac_reduce_scatter(ctxs(n), [b.ptr for b in sb], [b.ptr for b in rb], nb, dtype)
    run_and_check(rb, oracle.reduce_scatter(srcs, dtype), dtype, f"RS large misaligned {dtype}")


@pytest.mark.parametrize("aligned", [True, False], ids=["aligned", "dword-offsets"])
def test_large_tiles_allreduce_bf16_n8_rolling(ctxs, aligned):
    """The bf16 AllReduce of 8 ranks has its own kernel (a rolling load
    pipeline over the tile): buffers on the 16-byte grid, and sources 4, 8
    and 12 bytes off it (dword-aligned, so the rolling form still runs, with
    unaligned 16-byte loads), each with a ragged last tile."""
    n = 8
    m = 8 * (700_000 + 16) if aligned else 8 * (700_000 + 13)
    srcs = gen(n, m, "bf16", seed=47)
    nb = srcs[0].nbytes
    sb = [DevBuf(nb, offset=0 if aligned else 4 * (k % 4), data=s) for k, s in enumerate(srcs)]
    db = [DevBuf(nb, offset=0 if aligned else 8) for _ in srcs]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], nb, "bf16")
    run_and_check(db, oracle.all_reduce(srcs, "bf16"), "bf16", f"AR bf16 N=8 rolling aligned={aligned}")


@pytest.mark.parametrize("dtype", ["u32", "byte"])
def test_large_tiles_v_collectives(ctxs, dtype):
    n = 8
    m = 4_500_000 if dtype == "byte" else 1_200_000
    srcs = gen(n, m, dtype, seed=43)
    c = wl.v_counts(n, m, n, cfg=wl.CFG_TEST, seed=43)
    want = oracle.all_to_all_v(srcs, c)
    e = 4 if dtype == "u32" else 1
    sb = [DevBuf(s.nbytes, offset=e * (k % 3), data=s) for k, s in enumerate(srcs)]
    db = [DevBuf(np.asarray(w).nbytes, offset=e) for w in want]
    snac.snac_all_to_all_v(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], c.reshape(-1).tolist(), dtype)
    run_and_check(db, want, dtype, f"A2AV large {dtype}")
    row = c[0].tolist()
    gsrc = [gen(1, int(row[k]), dtype, seed=50 + k)[0] for k in range(n)]
    want = oracle.all_gather_v(gsrc, row)
    gb = [DevBuf(s.nbytes, data=s) for s in gsrc]
    db = [DevBuf(np.asarray(w).nbytes, offset=2 * e) for w in want]
    snac.snac_all_gather_v(ctxs(n), [b.ptr for b in gb], [b.ptr for b in db], row, dtype)
    run_and_check(db, want, dtype, f"AGV large {dtype}")


# One-to-one copies of 16 KiB tiles launch four workgroups per CU up to 8
# tiles per CU (2048 tiles on a 256-CU part: 32 MiB moved) and two beyond;
# these sizes sit inside that range, at its edge and just past it.
@pytest.mark.parametrize("per_rank", [1 << 20, 4 << 20, (4 << 20) + 2048])
def test_mid_size_all_to_all_launch_range(ctxs, per_rank):
    n = 8
    srcs = gen(n, per_rank // 4, "u32", seed=per_rank % 89)
    sb = [DevBuf(per_rank, offset=4 * (k % 2), data=s) for k, s in enumerate(srcs)]
    db = [DevBuf(per_rank, offset=16 * (k % 3)) for k in range(n)]
    snac.snac_all_to_all(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], per_rank, "u32")
    run_and_check(db, oracle.all_to_all(srcs), "u32", f"A2A {per_rank} B/rank")


# Reduces of at most 2 tiles per CU (4-8 MiB per rank on a 256-CU part)
# launch two workgroups per CU, larger ones one.
@pytest.mark.parametrize("per_rank", [(6 << 20) + 32, 8 << 20, (8 << 20) + 16384])
def test_mid_size_reduce_launch_range(ctxs, per_rank):
    n = 8
    srcs = gen(n, per_rank // 2, "bf16", seed=per_rank % 83)
    sb = [DevBuf(per_rank, data=s) for s in srcs]
    db = [DevBuf(per_rank, offset=16 * (k % 2)) for k in range(n)]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], per_rank, "bf16")
    run_and_check(db, oracle.all_reduce(srcs, "bf16"), "bf16", f"AR {per_rank} B/rank")
    rb = [DevBuf(per_rank // n) for _ in range(n)]
    snac.snac_reduce_scatter(ctxs(n), [b.ptr for b in sb], [b.ptr for b in rb], per_rank, "bf16")
    run_and_check(rb, oracle.reduce_scatter(srcs, "bf16"), "bf16", f"RS {per_rank} B/rank")


def test_mid_size_v_and_copy_launch_range(ctxs):
    n = 8
    m = (1 << 20) // 4  # 1 MiB of u32 per rank: about 512 tiles in all
    srcs = gen(n, m, "u32", seed=61)
    c = wl.v_counts(n, m, n, cfg=wl.CFG_TEST, seed=61)
    want = oracle.all_to_all_v(srcs, c)
    sb = [DevBuf(s.nbytes, data=s) for s in srcs]
    db = [DevBuf(np.asarray(w).nbytes, offset=4) for w in want]
    snac.snac_all_to_all_v(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], c.reshape(-1).tolist(), "u32")
    run_and_check(db, want, "u32", "A2AV 1 MiB/rank")
    nbytes = (12 << 20) + 5
    data = wl.raw_bytes(nbytes, wl.CFG_TEST, 0, seed=62)
    s = DevBuf(nbytes, offset=3, data=data)
    d = DevBuf(nbytes, offset=0)
    snac.snac_copy(d.ptr, s.ptr, nbytes)
    run_and_check([d], [oracle.copy(data)], "byte", "copy 12 MiB + 5 from a byte offset")


@pytest.mark.parametrize("per_rank", [256 * 16384 - 16, 256 * 16384, 256 * 16384 + 16])
def test_small_and_large_tiles_meet(ctxs, per_rank):
    """Sizes on both sides of the switch between the two tile sizes."""
    n = 8
    srcs = gen(n, per_rank // 2, "bf16", seed=per_rank % 97)
    sb = [DevBuf(per_rank, data=s) for s in srcs]
    db = [DevBuf(per_rank) for _ in srcs]
    snac.snac_all_reduce(ctxs(n), [b.ptr for b in sb], [b.ptr for b in db], per_rank, "bf16")
    run_and_check(db, oracle.all_reduce(srcs, "bf16"), "bf16", f"AR {per_rank} B/rank")
