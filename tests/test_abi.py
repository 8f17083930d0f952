"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, rejects invalid arguments before touching the GPU, and its layout
engine (snac_plan, the same code the kernels run) describes each collective
exactly: applying its jobs on the host reproduces the oracle."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "snac.h")


def declared_functions() -> list[str]:
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(snac_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = snac.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), f"{n} declared in snac.h but not exported"
    # and the binding wraps each of them under the same name
    for n in names:
        assert hasattr(snac, n), f"binding lacks {n}"


def test_nm_shows_c_linkage():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", snac.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (snac_\w+)", out))
    assert set(declared_functions()) <= exported


def test_versions_and_status_strings():
    assert snac.snac_abi_version() == 3
    for s in range(8):
        assert snac.snac_status_str(s).startswith("SNAC_")
    assert "unknown" in snac.snac_status_str(99)


def _expect(status, fn, *args):
    with pytest.raises(snac.SnacError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_argument_errors_without_gpu():
    E = snac.SNAC_E_ARG
    _expect(E, snac.snac_init, 0, 0)
    _expect(E, snac.snac_init, 17, 0)
    _expect(E, snac.snac_copy, 0, 0x1000, 16)
    _expect(E, snac.snac_copy, 0x1000, 0x1008, 16)  # overlap
    _expect(E, snac.snac_reduce_n, [0x1000], [0x2000], 8, "byte")
    _expect(E, snac.snac_reduce_n, [0x1000], [0x2000] * 17, 8, "f32")
    _expect(E, snac.snac_reduce_n, [0x1001], [0x2000], 8, "f32")  # misaligned
    _expect(E, snac.snac_reduce_n, [0x1000], [0x2000, 0x1010], 8, "f32")  # dst overlaps a src
    _expect(E, snac.snac_all_reduce, None, [0x1000], [0x2000], 16, "f32")
    _expect(E, snac.snac_check, None)
    _expect(E, snac.snac_abort, None)
    assert snac.snac_ctx_nranks(None) == 0
    # zero-size calls are no-ops, even with NULL pointers
    snac.snac_copy(0, 0, 0)
    snac.snac_reduce_n([0], [0], 0, "f32")
    snac.snac_finalize(None)


def test_probe_argument_errors_without_gpu():
    E = snac.SNAC_E_ARG

    def p(kind, dst, src, nbytes, threads=64, tile=4096, wgs=4):
        return lambda: snac.snac_hbm_probe(kind, dst, src, nbytes, threads, tile, wgs)

    _expect(E, p(7, 0x1000, 0x2000, 16))                 # unknown kind
    _expect(E, p(8 | 3, 0x1000, 0x2000, 16))             # unknown kind, ordered
    _expect(E, p("copy_ordered", 0x1008, 0x2000, 16))    # misaligned dst, ordered
    _expect(E, p("copy", 0x1000, 0x2000, 16, threads=128))  # workgroup size
    _expect(E, p("copy", 0x1000, 0x2000, 16, tile=8192))    # tile
    _expect(E, p("copy", 0x1000, 0x2000, 16, wgs=0))
    _expect(E, p("copy", 0x1000, 0x2000, 16, wgs=33))
    _expect(E, p("copy", 0x1000, 0x2000, 17))            # not whole 16-byte units
    _expect(E, p("copy", 0x1008, 0x2000, 16))            # misaligned dst
    _expect(E, p("read", 0x1000, 0x2004, 16))            # misaligned src
    _expect(E, p("copy", 0x1000, 0x1010, 64))            # overlap
    _expect(E, p("write", 0, None, 16))                  # no dst
    _expect(E, p("read", 0x1000, None, 16))              # no src
    _expect(E, p("copy", 0x1000, 1 << 44, snac.SNAC_MAX_BYTES + 16))  # past the size bound
    p("copy", 0, 0, 0)()                                 # nothing to do


def test_size_bound_without_gpu():
    """Extents and V counts above SNAC_MAX_BYTES are argument errors, so no
    extent or offset the checks compute can wrap; the bound itself passes
    the size check."""
    E, M = snac.SNAC_E_ARG, snac.SNAC_MAX_BYTES
    assert "SNAC_MAX_BYTES" in _expect(E, snac.snac_copy, 1 << 44, 0x1000, M + 1)
    assert "SNAC_MAX_BYTES" in _expect(E, snac.snac_copy, 1 << 44, 0x1000, (1 << 64) - 1)
    assert "SNAC_MAX_BYTES" in _expect(E, snac.snac_reduce_n, [1 << 44], [0x1000], M // 4 + 1, "f32")
    assert "SNAC_MAX_BYTES" in _expect(E, snac.snac_plan, snac.SNAC_COLL_ALL_REDUCE, 2, "f32", M + 4)
    assert "SNAC_MAX_BYTES" in _expect(E, snac.snac_plan, snac.SNAC_COLL_ALL_GATHER_V, 2, "byte", 0, [M + 1, 0])
    assert "SNAC_MAX_BYTES" in _expect(E, snac.snac_plan, snac.SNAC_COLL_ALL_TO_ALL_V, 2, "u32", 0,
                                       [1, 2, (1 << 64) - 1, 3])
    # at the bound the plan is made
    assert snac.snac_plan(snac.SNAC_COLL_ALL_REDUCE, 2, "bf16", M)[0][2] == M
    assert snac.snac_plan(snac.SNAC_COLL_ALL_GATHER_V, 2, "byte", 0, [M, 0])[0][2] == M


def test_static_atomic_allreduce_argument_errors_without_gpu():
    """The allocation-free AllReduce checks its arguments, its size limit
    included, before it touches the device."""
    E = snac.SNAC_E_ARG
    f = snac.snac_all_reduce_atomic_static
    _expect(E, f, [0x1000] * 17, [0x100000 * (i + 1) for i in range(17)], 64, "f32")   # too many ranks
    _expect(E, f, [0x1000, 0x2000], [0x3000, 0x4000], 64, "u32")                       # not a float type
    msg = _expect(E, f, [0x1000, 0x2000], [0x3000, 0x4000], ((1 << 23) + 1) * 4, "f32")  # past the scratch
    assert "static scratch" in msg
    _expect(E, f, [0x1000, 0x2000], [0x3000, 0x4000], 6, "f32")                        # not whole elements
    _expect(E, f, [0x1000, 0x1000], [0x3000, 0x3000], 64, "f32")                       # destinations overlap
    with pytest.raises(ValueError):
        f([0x1000], [0x3000, 0x4000], 64, "f32")
    f([0, 0], [0, 0], 0, "bf16")  # nothing to do


def test_tuning_roundtrip_and_ranges():
    t0 = snac.snac_get_tuning()
    try:
        snac.snac_set_tuning(wgs_per_cu=3, cache_policy=1)
        t = snac.snac_get_tuning()
        assert t["wgs_per_cu"] == 3 and t["cache_policy"] == 1
        _expect(snac.SNAC_E_ARG, lambda: snac.snac_set_tuning(cache_policy=9))
        _expect(snac.SNAC_E_ARG, lambda: snac.snac_set_tuning(pipeline_tile_bytes=1000))
        _expect(snac.SNAC_E_ARG, lambda: snac.snac_set_tuning(tile_schedule=3))
        snac.snac_set_tuning(tile_schedule=2)
        assert snac.snac_get_tuning()["tile_schedule"] == 2
    finally:
        snac.snac_set_tuning(**t0)


# ------------------------------------------------------------------ layouts
COLLS = {
    "all_reduce": snac.SNAC_COLL_ALL_REDUCE,
    "reduce_scatter": snac.SNAC_COLL_REDUCE_SCATTER,
    "all_gather": snac.SNAC_COLL_ALL_GATHER,
    "all_to_all": snac.SNAC_COLL_ALL_TO_ALL,
    "all_gather_v": snac.SNAC_COLL_ALL_GATHER_V,
    "reduce_scatter_v": snac.SNAC_COLL_REDUCE_SCATTER_V,
    "all_to_all_v": snac.SNAC_COLL_ALL_TO_ALL_V,
}


def apply_plan(jobs, srcs_bytes, out_sizes, dtype, n, esize):
    """Interpret a job list on the host: copy jobs move bytes, reduce jobs
    call the oracle's N-to-1 reduce on the element range.  Also checks that
    every output byte is written exactly once."""
    outs = [np.zeros(s, dtype=np.uint8) for s in out_sizes]
    written = [np.zeros(s, dtype=np.int32) for s in out_sizes]
    npd = {"f32": np.float32, "bf16": np.uint16}.get(dtype)
    for src_off, dst_off, nbytes, sr, dr in jobs:
        assert nbytes > 0 and nbytes % esize == 0 and src_off % esize == 0 and dst_off % esize == 0
        if sr < 0:
            parts = [s[src_off:src_off + nbytes].view(npd) for s in srcs_bytes]
            data = oracle.reduce_n(parts, dtype).view(np.uint8)
        else:
            assert src_off + nbytes <= srcs_bytes[sr].size
            data = srcs_bytes[sr][src_off:src_off + nbytes]
        targets = range(n) if dr < 0 else [dr]
        for d in targets:
            assert dst_off + nbytes <= out_sizes[d]
            outs[d][dst_off:dst_off + nbytes] = data
            written[d][dst_off:dst_off + nbytes] += 1
    for w in written:
        assert np.all(w == 1), "an output byte was written zero or several times"
    return outs


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("name", sorted(COLLS))
def test_plan_matches_oracle(name, n):
    dtype = "bf16" if "reduce" in name else "u32"
    esize = 2 if dtype == "bf16" else 4
    g = np.random.default_rng(n)
    if name in ("all_reduce", "all_gather"):
        m = 37
        srcs = [wl.raw_bytes(m * esize, wl.CFG_TEST, r) for r in range(n)]
        jobs = snac.snac_plan(COLLS[name], n, dtype, m * esize)
        if name == "all_reduce":
            want = oracle.all_reduce([s.view(np.uint16) for s in srcs], "bf16")
            sizes = [m * esize] * n
        else:
            want = oracle.all_gather(srcs)
            sizes = [n * m * esize] * n
    elif name in ("reduce_scatter", "all_to_all"):
        m = 6 * n
        srcs = [wl.raw_bytes(m * esize, wl.CFG_TEST, r) for r in range(n)]
        jobs = snac.snac_plan(COLLS[name], n, dtype, m * esize)
        if name == "reduce_scatter":
            want = oracle.reduce_scatter([s.view(np.uint16) for s in srcs], "bf16")
            sizes = [m // n * esize] * n
        else:
            want = oracle.all_to_all(srcs)
            sizes = [m * esize] * n
    elif name == "all_to_all_v":
        c = g.integers(0, 6, size=(n, n))
        c[0, 0] = 0
        srcs = [wl.raw_bytes(int(c[s].sum()) * esize, wl.CFG_TEST, s) for s in range(n)]
        jobs = snac.snac_plan(COLLS[name], n, dtype, 0, c.reshape(-1).tolist())
        want = oracle.all_to_all_v([s.view(np.uint32) for s in srcs], c)
        sizes = [int(c[:, d].sum()) * esize for d in range(n)]
    else:
        c = g.integers(0, 6, size=n)
        c[-1] = 0
        tot = int(c.sum())
        jobs = snac.snac_plan(COLLS[name], n, dtype, 0, c.tolist())
        if name == "all_gather_v":
            srcs = [wl.raw_bytes(int(c[k]) * esize, wl.CFG_TEST, k) for k in range(n)]
            want = oracle.all_gather_v([s.view(np.uint32) for s in srcs], list(c))
            sizes = [tot * esize] * n
        else:
            srcs = [wl.raw_bytes(tot * esize, wl.CFG_TEST, k) for k in range(n)]
            want = oracle.reduce_scatter_v([s.view(np.uint16) for s in srcs], list(c), "bf16")
            sizes = [int(x) * esize for x in c]
    outs = apply_plan(jobs, srcs, sizes, dtype, n, esize)
    for o, w in zip(outs, want):
        assert np.array_equal(o, np.asarray(w).view(np.uint8))


def test_plan_rejects_bad_requests():
    E = snac.SNAC_E_ARG
    _expect(E, snac.snac_plan, snac.SNAC_COLL_REDUCE_SCATTER, 3, "f32", 16)  # not N*e divisible
    _expect(E, snac.snac_plan, snac.SNAC_COLL_ALL_REDUCE, 2, "byte", 16)      # reduce needs floats
    _expect(E, snac.snac_plan, snac.SNAC_COLL_ALL_REDUCE, 0, "f32", 16)
    _expect(E, snac.snac_plan, 42, 2, "f32", 16)
    _expect(E, snac.snac_plan, snac.SNAC_COLL_ALL_TO_ALL_V, 2, "f32", 0, None)
    # more jobs than room
    with pytest.raises(snac.SnacError):
        snac.snac_plan(snac.SNAC_COLL_ALL_TO_ALL, 4, "f32", 64, max_jobs=3)


# ------------------------------------------------------- device-side API
def test_device_api_argument_errors_without_gpu():
    E = snac.SNAC_E_ARG
    _expect(E, snac.snac_get_device_context, None)
    _expect(E, snac.snac_describe, None, snac.SNAC_COLL_ALL_REDUCE, [0x1000], [0x2000], 16, None, "f32")


def _c_layout(struct: str, fields: list[str]) -> list[int]:
    """sizeof and offsetof of a snac.h struct as the C compiler lays it out."""
    import subprocess
    import tempfile

    body = "\n".join(f'  printf("%zu\\n", offsetof({struct}, {f}));' for f in fields)
    src = f'#include <stddef.h>\n#include <stdio.h>\n#include "snac.h"\nint main(void) {{\n' \
          f'  printf("%zu\\n", sizeof({struct}));\n{body}\n  return 0;\n}}\n'
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        return [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]


@pytest.mark.parametrize("cls", [snac.snac_dev_ctx, snac.snac_coll_desc, snac.snac_tuning, snac.snac_job])
def test_binding_structs_match_c_layout(cls):
    names = [n for n, _ in cls._fields_]
    got = _c_layout(cls.__name__, names)
    assert got[0] == ctypes.sizeof(cls)
    for n, off in zip(names, got[1:]):
        assert getattr(cls, n).offset == off, n
    if cls is snac.snac_coll_desc:
        assert ctypes.sizeof(cls) == 2336  # as documented in snac.h


def test_devtest_fixture_exports_its_launchers():
    lib = ctypes.CDLL(os.path.join(ROOT, "tests", "devapi", "libsnac_devtest.so"))
    for n in ("devtest_copy_slices", "devtest_reduce_slices", "devtest_collective", "devtest_collective_nosync",
              "devtest_fused_scale_allreduce", "devtest_flags", "devtest_many_flags"):
        assert hasattr(lib, n)


# ------------------------------------------------------------ tuning rules
def test_builtin_tuning_rules_and_lookup():
    snac.snac_set_tuning_rules(None)
    rules = snac.snac_get_tuning_rules()
    assert len(rules) >= 3
    MiB = 1 << 20
    # measured defaults: reduces and copies keep the kernel's workgroups per CU
    # (0: it depends on the tile size and source count), streaming accesses
    for coll, n, e, b in ((snac.SNAC_COLL_ALL_REDUCE, 8, 2, 256 * MiB), (snac.SNAC_COLL_REDUCE_SCATTER, 4, 4, 1),
                          (snac.SNAC_COLL_REDUCE_SCATTER_V, 8, 4, 1),
                          (snac.SNAC_RULE_ATOM_REDUCE, 2, 4, 1), (snac.SNAC_COLL_ALL_GATHER, 8, 1, 1),
                          (snac.SNAC_COLL_ALL_TO_ALL, 8, 4, 64 * MiB), (snac.SNAC_RULE_ATOM_COPY, 1, 1, MiB)):
        assert snac.snac_tuning_lookup(coll, n, e, b)["wgs_per_cu"] == 0, coll
    assert snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_REDUCE, 8, 2, 256 * MiB)["cache_policy"] == 1
    # AllGather(V) reads inputs with cached loads (streaming stores)
    assert snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_GATHER_V, 8, 2, 1)["cache_policy"] == 2
    assert snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_TO_ALL, 8, 4, 1)["cache_policy"] == 1
    assert snac.snac_tuning_lookup(snac.SNAC_RULE_ATOM_COPY, 1, 1, 1)["cache_policy"] == 1
    # the pipeline: one WG per CU at every size
    assert snac.snac_tuning_lookup(snac.SNAC_RULE_PIPELINE, 8, 2, MiB)["wgs_per_cu"] == 1
    assert snac.snac_tuning_lookup(snac.SNAC_RULE_PIPELINE, 8, 2, 64 * MiB)["wgs_per_cu"] == 1


def test_tuning_rules_first_match_and_override():
    MiB = 1 << 20
    try:
        snac.snac_set_tuning_rules([
            {"coll": snac.SNAC_COLL_ALL_REDUCE, "min_ranks": 8, "max_ranks": 8, "esize": 2, "min_bytes": 0,
             "max_bytes": MiB, "wgs_per_cu": 4, "cache_policy": 4},
            {"coll": snac.SNAC_RULE_ANY_REDUCE, "min_ranks": 1, "max_ranks": 16, "esize": 0, "min_bytes": 0,
             "max_bytes": 2 ** 64 - 1, "wgs_per_cu": 3, "cache_policy": 2},
        ])
        assert len(snac.snac_get_tuning_rules()) == 2
        t = snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_REDUCE, 8, 2, MiB)
        assert (t["wgs_per_cu"], t["cache_policy"]) == (4, 4)
        t = snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_REDUCE, 8, 2, MiB + 1)  # past the first rule's range
        assert (t["wgs_per_cu"], t["cache_policy"]) == (3, 2)
        t = snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_REDUCE, 8, 4, 16)  # f32: first rule wants esize 2
        assert (t["wgs_per_cu"], t["cache_policy"]) == (3, 2)
        t = snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_TO_ALL, 8, 4, 16)  # no rule: kernel defaults
        assert (t["wgs_per_cu"], t["cache_policy"]) == (0, 0)
        snac.snac_set_tuning(wgs_per_cu=5)  # explicit process-wide value wins
        assert snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_REDUCE, 8, 2, 64)["wgs_per_cu"] == 5
    finally:
        snac.snac_set_tuning(wgs_per_cu=0)
        snac.snac_set_tuning_rules(None)
    assert len(snac.snac_get_tuning_rules()) >= 3


@pytest.mark.parametrize("bad", [
    {"coll": 7}, {"coll": -4}, {"min_ranks": 0}, {"min_ranks": 5, "max_ranks": 4}, {"max_ranks": 17},
    {"esize": 3}, {"min_bytes": 10, "max_bytes": 9}, {"wgs_per_cu": 33}, {"cache_policy": 5},
])
def test_invalid_tuning_rules_rejected(bad):
    good = {"coll": -1, "min_ranks": 1, "max_ranks": 16, "esize": 0, "min_bytes": 0, "max_bytes": 100,
            "wgs_per_cu": 1, "cache_policy": 1}
    before = snac.snac_get_tuning_rules()
    _expect(snac.SNAC_E_ARG, snac.snac_set_tuning_rules, [good, {**good, **bad}])
    assert snac.snac_get_tuning_rules() == before  # unchanged on error


def test_reduce_mode_argument_errors_without_gpu():
    _expect(snac.SNAC_E_ARG, snac.snac_all_reduce_ex, None, [0x1000], [0x2000], 16, "f32", "atomic")
    _expect(snac.SNAC_E_ARG, snac.snac_all_reduce_ex, None, [0x1000], [0x2000], 16, "f32", 7)


def test_tuning_from_environment():
    """SNAC_* variables seed the process-wide tuning; invalid ones are ignored."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r); import copy_reduce_snac_amd as s; t = s.snac_get_tuning(); "
            "print(t['wgs_per_cu'], t['cache_policy'], t['pipeline_tile_bytes'], t['spin_limit_log2'], "
            "t['copy_multicast'], t['tile_schedule'])" % ROOT)
    env = dict(os.environ, SNAC_WGS_PER_CU="3", SNAC_CACHE_POLICY="4", SNAC_PIPELINE_TILE_BYTES="8192",
               SNAC_SPIN_LIMIT_LOG2="99", SNAC_COPY_MULTICAST="x1", SNAC_TILE_SCHEDULE="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True).stdout
    assert out.split() == ["3", "4", "8192", "0", "0", "1"]
    env["SNAC_TILE_SCHEDULE"] = "5"
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True).stdout
    assert out.split()[-1] == "0"


def test_binding_refuses_rank_lists_of_the_wrong_length(monkeypatch):
    """The library reads exactly N pointers (and N or N*N counts) per call,
    so the binding checks every per-rank list against the context's rank
    count before calling it.  A stand-in rank count for a fake context keeps
    this on the CPU: the refusals happen before any library call."""
    monkeypatch.setattr(snac, "snac_ctx_nranks", lambda ctx: 4)
    fake = 0x1000
    four, three = [0x10000] * 4, [0x10000] * 3
    calls = [
        lambda: snac.snac_all_reduce(fake, three, four, 64, "f32"),
        lambda: snac.snac_reduce_scatter(fake, four, three, 64, "f32"),
        lambda: snac.snac_all_gather(fake, four, [0x10000] * 5, 64, "f32"),
        lambda: snac.snac_all_to_all(fake, [], four, 64, "u32"),
        lambda: snac.snac_all_reduce_ex(fake, four, three, 64, "bf16", "atomic"),
        lambda: snac.snac_all_gather_v(fake, four, four, [1, 2, 3], "u32"),
        lambda: snac.snac_reduce_scatter_v(fake, four, four, [1] * 5, "f32"),
        lambda: snac.snac_all_to_all_v(fake, four, four, [1] * 4, "u32"),
        lambda: snac.snac_pipeline_scale_reduce(fake, three, 0x10000, 16, "bf16"),
        lambda: snac.snac_describe(fake, snac.SNAC_COLL_ALL_REDUCE, three, four, 64, None, "f32"),
        lambda: snac.snac_describe(fake, snac.SNAC_COLL_ALL_TO_ALL_V, four, four, 0, [1] * 4, "u32"),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call()


def test_tuning_tables_survive_concurrent_use():
    """The rule table and the process-wide tuning are read by every call and
    may be replaced from another host thread meanwhile: a reader must always
    see one whole table (ctypes releases the GIL around library calls, so
    the threads really overlap)."""
    import threading

    MiB = 1 << 20
    table_a = [{"coll": snac.SNAC_COLL_ALL_REDUCE, "min_ranks": 1, "max_ranks": 16, "esize": 0, "min_bytes": 0,
                "max_bytes": 2 ** 64 - 1, "wgs_per_cu": 3, "cache_policy": 2}]
    table_b = [{"coll": snac.SNAC_RULE_ANY, "min_ranks": 1, "max_ranks": 16, "esize": 0, "min_bytes": 0,
                "max_bytes": MiB, "wgs_per_cu": 5, "cache_policy": 4}] * 40 + table_a
    seen, errors = set(), []
    stop = threading.Event()

    def writer():
        try:
            for i in range(3000):
                snac.snac_set_tuning_rules(table_a if i % 2 else table_b)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)
        finally:
            stop.set()

    def reader():
        try:
            while not stop.is_set():
                t = snac.snac_tuning_lookup(snac.SNAC_COLL_ALL_REDUCE, 8, 2, 4 * MiB)
                seen.add((t["wgs_per_cu"], t["cache_policy"]))
                n = len(snac.snac_get_tuning_rules())
                assert n in (1, 41), n
        except Exception as e:
            errors.append(e)

    threads = [threading.Thread(target=writer)] + [threading.Thread(target=reader) for _ in range(3)]
    try:
        for t in threads:
            t.start()
        for t in threads:
            t.join()
    finally:
        snac.snac_set_tuning_rules(None)
    assert not errors, errors
    assert seen <= {(3, 2)}, seen  # 4 MiB is past table B's first 40 rules: both tables give (3, 2)


def test_kernel_hash_ignores_comments_only():
    """bench.py reports counter-based traffic only while the counters match
    the kernel sources; comments and layout must not count as changes."""
    import sys

    sys.path.insert(0, ROOT)
    import bench

    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x /*y*/";  char q = \'"\';\n'
    assert bench.code_only(src) == 'int a = 1; const char* s = "//x /*y*/"; char q = \'"\';'
    assert bench.code_only("a  +\n\tb") == bench.code_only("a + b")
    assert bench.code_only("a + b") != bench.code_only("a - b")
    assert len(bench.kernel_source_hash()) == 16
