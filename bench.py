"""Benchmark of the copy / N-to-1 reduce collective datapath on one MI355X.

Default run (the headline): AllReduce(sum) over N = 8 logical ranks, bf16
inputs with binary32 accumulation and bf16 output, 256 MiB per rank, the
result written to all 8 destination buffers.  A step is one AllReduce call
(one kernel) over inputs already resident in HBM.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--jsonl PATH]

Prints one JSON line.  ``value`` is the algorithmic HBM bandwidth of the
AllReduce, 2 * N * B bytes per call (every source read once, every
destination written once) over the mean time of exactly --steps calls
timed with HIP events on the launch stream.  ``roofline`` relates that to
the 8 TB/s HBM peak and to the 1:1 read/write (copy) ceiling measured in
the same run; ``traffic`` is the HBM traffic per launch from rocprofv3
counters when the recorded counters match the current kernel sources
(else null).  ``cpu_baseline`` times the CPU oracle on a bounded sample of
the same workload.  ``extra`` holds, each measured the same way and with
the counter figures of its own summary when valid:

  * the other configured workloads (ReduceScatter then AllGather, AllToAll,
    AllToAllV, AllGatherV, ReduceScatterV, the SNAC pipeline in bf16 and
    f32 and its latency sizes, a 1 GiB copy, the atomic AllReduce mode);
  * the HBM ceilings (read-only, write-only, 1:1 copy probes);
  * the AllReduce sweep, 1 KiB .. 1 GiB per rank, and the AllGather sweep,
    128 B .. 128 MiB in per rank, each size the median over 20 runs of a
    HIP graph of 10 calls (1 call from 64 MiB per rank up).  A row is
    cache_resident when its whole working set fits the 256 MB Infinity
    Cache, inputs_cache_resident when its inputs do (so that replays read
    them from there).

Per collective, in the argument form of the pages' benchmark binaries:

    python bench.py --coll NAME [minBytes [maxBytes [graphLaunches [runs [warmup [seed]]]]]]
                    [--dtype D] [--nranks N] [--jsonl PATH]

NAME is allreduce, reduce_scatter, all_gather, all_to_all, all_gather_v,
reduce_scatter_v or all_to_all_v (or AR, RS, AG, A2A, AGV, RSV, A2AV).
Sizes take K, M and G (powers of 1024) and double from minBytes to
maxBytes; a size is the per-rank input (for AllGather: per-rank input, for
the V variants: the per-rank total of the counts).  Each size is a HIP
graph of graphLaunches calls replayed `runs` times after `warmup` replays;
the median per call is reported, one JSON line per size (also appended to
--jsonl).  algbw uses the pages' totalBytes: the output size for
AllGather(V), the per-rank input size otherwise.

Single workloads for profiler runs:

    python bench.py --only NAME [--steps K] [--warmup W]

NAME: allreduce, allreduce_atomic, copy, rs, ag, ag_cold, rs_ag, a2a, a2av,
agv, rsv, pipeline_bf16, pipeline_f32, pipeline_latency, ceilings,
sweep_ar, sweep_ag.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s & % of peak, 8-logical-rank bf16 AllReduce reduceN, 256 MiB/rank"
PEAK_GBPS = 8000.0
KiB = 1 << 10
MiB = 1 << 20
GiB = 1 << 30
N = 8
INFINITY_CACHE = 256 * MiB
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------- kernel-source hashes
# Counter summaries record the hash of the sources of the kernels they
# measured; a summary whose hash differs from the current sources is stale
# and its figures are not reported.
_COMMON = ("include/snac_device.hpp", "include/snac_layout.hpp", "include/snac.h",
           "copy_reduce_snac_amd/csrc/internal.hpp")
KERNEL_SOURCES = _COMMON + ("copy_reduce_snac_amd/csrc/collectives.hip",)
SOURCE_SETS = {
    "collectives": KERNEL_SOURCES,
    "pipeline": _COMMON + ("copy_reduce_snac_amd/csrc/pipeline.hip",),
    "probes": _COMMON + ("copy_reduce_snac_amd/csrc/probes.hip",),
}


def code_only(src: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed,
    so that edits to comments or layout alone do not count as kernel
    changes.  String and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(names=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return source_hash(KERNEL_SOURCES)


def read_counter_summaries() -> dict:
    """Machine-readable lines ("- key: `value`") of every profiles/*_counters.md,
    keyed by its `workload` value; only summaries whose kernel_source_hash
    matches the current sources of their `sources` set."""
    out = {}
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_counters.md"))):
        vals = {}
        for line in open(path, encoding="utf-8").read().splitlines():
            m = re.match(r"\s*- ([a-z_0-9]+): `([^`]*)`", line)
            if m:
                vals[m.group(1)] = m.group(2)
        key, srcs = vals.get("workload"), vals.get("sources", "collectives")
        if not key or srcs not in SOURCE_SETS:
            continue
        if vals.get("kernel_source_hash") != source_hash(SOURCE_SETS[srcs]):
            continue
        vals["file"] = os.path.relpath(path, ROOT)
        out[key] = vals
    return out


COUNTERS: dict = {}


def attach_counters(row: dict, key: str) -> dict:
    """Add the counter figures of summary `key` (traffic per launch, its
    ratio to the algorithmic bytes, L2 hit rate) when it is valid."""
    c = COUNTERS.get(key)
    row["counters"] = key
    if not c:
        row["traffic_bytes"] = None
        return row
    try:
        tr = float(c["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        tr = None
    row["traffic_bytes"] = tr
    if tr and row.get("algorithmic_bytes"):
        row["traffic_over_algorithmic"] = round(tr / row["algorithmic_bytes"], 5)
    if "l2_hit" in c:
        row["l2_hit"] = float(c["l2_hit"])
    row["counters_file"] = c["file"]
    return row


# ------------------------------------------------------------------ timing
class Env:
    def __init__(self):
        import torch

        import copy_reduce_snac_amd as snac

        self.torch = torch
        self.snac = snac
        snac.lib()  # fail loudly if the library is missing
        torch.cuda.set_device(0)
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        self.ctx = snac.snac_init(N, 0, self.stream)

    def upload(self, a: np.ndarray):
        t = self.torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1))
        return t.to(self.dev, non_blocking=False)

    def empty(self, nbytes: int):
        return self.torch.empty(max(1, nbytes), dtype=self.torch.uint8, device=self.dev)

    def time_calls(self, fn, steps: int, warmup: int) -> float:
        """Seconds per call: events on the launch stream around exactly
        `steps` calls, after `warmup` untimed ones."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(steps):
            fn()
        end.record(self.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / 1e3 / steps

    def time_calls_cold(self, fn, steps: int, warmup: int) -> float:
        """Seconds per call with the inputs evicted from the caches first: a
        1 GiB scratch buffer is read (untimed) before each event-timed call.
        A read, not a write: a write would leave the Infinity Cache full of
        dirty lines whose write-back the timed call would then pay for."""
        torch = self.torch
        scratch = torch.ones(1 << 27, dtype=torch.int64, device=self.dev)
        for _ in range(warmup):
            fn()
        total = 0.0
        for _ in range(steps):
            scratch.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1) / 1e3
        del scratch
        return total / steps

    def graph_median(self, call, batch: int = 10, runs: int = 20, warmup: int = 5) -> float:
        """Median seconds per call: `batch` calls captured in one HIP graph
        (call(stream) launches one), replayed `warmup` times untimed, then
        `runs` times, each replay timed with events."""
        torch = self.torch
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            call(torch.cuda.current_stream())  # first launch outside the capture
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for _ in range(batch):
                    call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(runs):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3 / batch)
        del g
        return float(np.median(times))


def result(name, t, alg_bytes, total_bytes, **kw):
    d = {
        "workload": name,
        "ms_per_call": round(t * 1e3, 5),
        "algbw_GBps": round(total_bytes / t / 1e9, 2),
        "hbm_GBps": round(alg_bytes / t / 1e9, 2),
        "frac_of_peak": round(alg_bytes / t / 1e9 / PEAK_GBPS, 4),
        "algorithmic_bytes": int(alg_bytes),
        "total_bytes": int(total_bytes),
    }
    d.update(kw)
    return d


def gen_bf16(m: int, cfg: int, rank: int, seed: int = 0) -> np.ndarray:
    from copy_reduce_snac_amd import workloads as wl

    return wl.normal_bf16(m, cfg, rank, seed=seed)


# -------------------------------------------------------- collective specs
# For a per-rank size B (bytes) and N ranks: per-rank output bytes, the
# algorithmic bytes of one call (every byte read once and written once, as
# the layout moves them), and the pages' totalBytes.
SPECS = {
    "allreduce": dict(dtype="bf16", out=lambda B, n: B, alg=lambda B, n: 2 * n * B, total=lambda B, n: B),
    "reduce_scatter": dict(dtype="bf16", out=lambda B, n: B // n, alg=lambda B, n: n * B + B, total=lambda B, n: B),
    "all_gather": dict(dtype="bf16", out=lambda B, n: n * B, alg=lambda B, n: n * B + n * n * B,
                       total=lambda B, n: n * B),
    "all_to_all": dict(dtype="u32", out=lambda B, n: B, alg=lambda B, n: 2 * n * B, total=lambda B, n: B),
    "all_gather_v": dict(dtype="u32", out=lambda B, n: B, alg=lambda B, n: B + n * B, total=lambda B, n: B),
    "reduce_scatter_v": dict(dtype="f32", out=None, alg=lambda B, n: n * B + B, total=lambda B, n: B),
    "all_to_all_v": dict(dtype="u32", out=None, alg=lambda B, n: 2 * n * B, total=lambda B, n: B),
}
ALIASES = {"AR": "allreduce", "RS": "reduce_scatter", "AG": "all_gather", "A2A": "all_to_all",
           "AGV": "all_gather_v", "RSV": "reduce_scatter_v", "A2AV": "all_to_all_v", "all_reduce": "allreduce"}
ESIZE = {"bf16": 2, "f32": 4, "u32": 4, "byte": 1}


def parse_size(s: str) -> int:
    m = re.fullmatch(r"\s*(\d+)\s*([KMG]?)i?B?\s*", s, flags=re.I)
    if not m:
        raise SystemExit(f"bad size {s!r}: use e.g. 1K, 128M, 1G or a byte count")
    return int(m.group(1)) << {"": 0, "K": 10, "M": 20, "G": 30}[m.group(2).upper()]


class Sweep:
    """Inputs for one collective at sizes up to `top` bytes per rank, and a
    call(size, stream) that runs the collective at any of them (prefixes of
    the same seeded buffers; V counts drawn per size)."""

    def __init__(self, env: Env, coll: str, top: int, dtype: str, n: int, seed: int):
        from copy_reduce_snac_amd import workloads as wl

        self.env, self.coll, self.n, self.dtype, self.seed = env, coll, n, dtype, seed
        self.e = ESIZE[dtype]
        snac = env.snac
        self.snac = snac
        self.ctx = env.ctx if n == N else snac.snac_init(n, 0, env.stream)
        cfg = {"allreduce": wl.CFG_AR_BF16_N8, "reduce_scatter": wl.CFG_RS_AG_BF16_N8,
               "all_gather": wl.CFG_RS_AG_BF16_N8}.get(coll, wl.CFG_A2A_N8)
        elems = top // self.e
        t0 = time.time()
        if dtype == "bf16":
            host = [wl.normal_bf16(elems, cfg, r, seed=seed) for r in range(n)]
        elif dtype == "f32":
            host = [wl.normal_f32(elems, cfg, r, seed=seed) for r in range(n)]
        elif dtype == "u32":
            host = [wl.raw_u32(elems, cfg, r, seed=seed) for r in range(n)]
        else:
            host = [wl.raw_bytes(elems, cfg, r, seed=seed) for r in range(n)]
        self.src = [env.upload(h) for h in host]
        del host
        out = SPECS[coll]["out"]
        self.dst = [env.empty(out(top, n) if out else top) for _ in range(n)]
        self.cfg = cfg
        log(f"{coll}: {n} x {top} B inputs ready in {time.time() - t0:.1f}s")

    def close(self):
        if self.ctx != self.env.ctx:
            self.snac.snac_finalize(self.ctx, self.env.stream)
        del self.src, self.dst

    def call_for(self, B: int):
        """A call(stream) running the collective at B bytes per rank."""
        from copy_reduce_snac_amd import workloads as wl

        snac, ctx, src, dst, dt, n = self.snac, self.ctx, self.src, self.dst, self.dtype, self.n
        c = self.coll
        if c == "allreduce":
            return lambda st: snac.snac_all_reduce(ctx, src, dst, B, dt, st)
        if c == "reduce_scatter":
            return lambda st: snac.snac_reduce_scatter(ctx, src, dst, B, dt, st)
        if c == "all_gather":
            return lambda st: snac.snac_all_gather(ctx, src, dst, B, dt, st)
        if c == "all_to_all":
            return lambda st: snac.snac_all_to_all(ctx, src, dst, B, dt, st)
        E = B // self.e
        if c == "all_to_all_v":
            counts = wl.v_counts(n, E, n, cfg=self.cfg, seed=self.seed).reshape(-1).tolist()
            return lambda st: snac.snac_all_to_all_v(ctx, src, dst, counts, dt, st)
        row = wl.v_counts(n, E, 1, cfg=self.cfg, seed=self.seed)[0].tolist()
        if c == "all_gather_v":
            return lambda st: snac.snac_all_gather_v(ctx, src, dst, row, dt, st)
        return lambda st: snac.snac_reduce_scatter_v(ctx, src, dst, row, dt, st)


def sweep_rows(env: Env, coll: str, lo: int, hi: int, graph_launches: int | None, runs: int, warmup: int, seed: int,
               dtype: str | None = None, n: int = N, jsonl=None, emit=False):
    """One row per size lo, 2 lo, ..., hi.  graph_launches None: 10 calls
    per graph below 64 MiB per rank, 1 from there up."""
    spec = SPECS[coll]
    dtype = dtype or spec["dtype"]
    sw = Sweep(env, coll, hi, dtype, n, seed)
    rows = []
    B = lo
    try:
        while B <= hi:
            K = graph_launches if graph_launches else (10 if B < 64 * MiB else 1)
            t = env.graph_median(sw.call_for(B), batch=K, runs=runs, warmup=warmup)
            alg = spec["alg"](B, n)
            inputs = n * (B if coll != "all_gather_v" else B // n)
            r = result(f"{coll} {dtype} N={n} {B} B/rank", t, alg, spec["total"](B, n), collective=coll,
                       dtype=dtype, nranks=n, bytes_per_rank=B,
                       timing=f"median over {runs} runs of a HIP graph of {K} calls",
                       cache_resident=bool(alg < INFINITY_CACHE),
                       inputs_cache_resident=bool(inputs < INFINITY_CACHE), seed=seed)
            rows.append(r)
            if emit:
                print(json.dumps(r), flush=True)
            if jsonl:
                jsonl.write(json.dumps(r) + "\n")
                jsonl.flush()
            B *= 2
    finally:
        sw.close()
        env.torch.cuda.empty_cache()
    return rows


# ---------------------------------------------------------------- workloads
def run_allreduce(env: Env, steps: int, warmup: int, per_rank: int = 256 * MiB, cpu: bool = True,
                  top: int = 256 * MiB, graph: bool = True):
    """The headline.  Inputs are the first `per_rank` bytes of seeded
    buffers of `top` bytes per rank (the same values at any top)."""
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    t0 = time.time()
    host = [gen_bf16(top // 2, wl.CFG_AR_BF16_N8, r) for r in range(N)]
    src = [env.upload(h) for h in host]
    dst = [env.empty(top) for _ in range(N)]
    log(f"allreduce: inputs ready in {time.time() - t0:.1f}s")

    def call():
        snac.snac_all_reduce(env.ctx, src, dst, per_rank, "bf16", env.stream)

    t = env.time_calls(call, steps, warmup)
    alg = 2 * N * per_rank
    out = result(f"allreduce_sum bf16 N={N} {per_rank // MiB} MiB/rank", t, alg, per_rank,
                 timing=f"mean of {steps} calls after {warmup} warmup calls")
    if graph:
        # the same calls as the pages' benchmark times them: median over 20
        # runs of a one-call HIP graph
        out["graph_median_ms"] = round(env.graph_median(
            lambda st: snac.snac_all_reduce(env.ctx, src, dst, per_rank, "bf16", st), batch=1, runs=20,
            warmup=5) * 1e3, 5)
    cpu_res = None
    if cpu:
        cpu_res = cpu_baseline_allreduce([h[:per_rank // 2] for h in host], dst, per_rank)
    del src, dst, host
    env.torch.cuda.empty_cache()
    return attach_counters(out, "allreduce"), cpu_res


def run_allreduce_atomic(env: Env, steps: int, warmup: int, per_rank: int = 256 * MiB):
    """The non-deterministic (float-atomic) AllReduce mode on the headline
    workload, for comparison with the deterministic kernel."""
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    m = per_rank // 2
    src = [env.upload(gen_bf16(m, wl.CFG_AR_BF16_N8, r)) for r in range(N)]
    dst = [env.empty(per_rank) for _ in range(N)]
    # accumulator: a staging ring per rank big enough for the binary32 sums
    ctx = snac.snac_init(N, 2 * per_rank // N, env.stream)
    try:
        t = env.time_calls(lambda: snac.snac_all_reduce_ex(ctx, src, dst, per_rank, "bf16", "atomic", env.stream),
                           steps, warmup)
    finally:
        snac.snac_finalize(ctx, env.stream)
    return result(f"allreduce_sum bf16 N={N} {per_rank // MiB} MiB/rank, atomic (non-deterministic) mode", t,
                  2 * N * per_rank, per_rank)


def host_info() -> dict:
    """CPU model, host RAM and thread counts of the machine running this."""
    model, mem = "unknown", None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal:"):
                mem = round(int(line.split()[1]) / (1 << 20), 1)
                break
    except OSError:
        pass
    return {"host_cpu_model": model, "host_mem_GiB": mem, "nproc": os.cpu_count(),
            "host_threads_available": len(os.sched_getaffinity(0))}


def cpu_baseline_allreduce(host, dst, per_rank, budget_s: float = 10.0):
    """The oracle, as it stands, over consecutive 32 MiB-per-rank slices of
    the same inputs, cycling through the whole workload until about
    `budget_s` seconds of CPU time have been spent.  The first pass also
    checks the GPU output slice by slice."""
    import oracle

    m = per_rank // 2
    slice_elems = 16 * MiB
    done = 0  # elements reduced, over every pass
    spent = 0.0
    ok = True
    got = dst[0][:per_rank].cpu().numpy().view(np.uint16)
    passes = 0
    while spent < budget_s:
        lo = done % m
        hi = min(m, lo + slice_elems)
        parts = [h[lo:hi] for h in host]
        t0 = time.perf_counter()
        want = oracle.reduce_n(parts, "bf16")
        spent += time.perf_counter() - t0
        if passes == 0:
            ok = ok and bool(np.array_equal(got[lo:hi], want))
        done += hi - lo
        if hi == m:
            passes += 1
    value = 2 * N * done * 2 / spent / 1e9
    res = {
        "value": round(value, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole 256 MiB-per-rank workload in 32 MiB slices, cycled {done / m:.1f} times "
                  f"(NumPy, single thread, {spent:.1f} s); GPU output equal on the first pass: {ok}",
        "parallel": cpu_baseline_allreduce_threads(host, m),
    }
    res.update(host_info())
    return res


def cpu_baseline_allreduce_threads(host, m: int, budget_s: float = 3.0):
    """The same oracle call on P threads at once, each over its own slices of
    the element range (NumPy releases the GIL inside its loops), whole passes
    over the workload until about `budget_s` seconds of wall time."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    slice_elems = 4 * MiB
    bounds = [(lo, min(m, lo + slice_elems)) for lo in range(0, m, slice_elems)]

    def work(k):
        for lo, hi in bounds[k::threads]:
            oracle.reduce_n([h[lo:hi] for h in host], "bf16")

    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as pool:
        while passes == 0 or time.perf_counter() - t0 < budget_s:
            list(pool.map(work, range(threads)))
            passes += 1
    wall = time.perf_counter() - t0
    return {
        "value": round(2 * N * m * 2 * passes / wall / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "sample": f"{passes} whole passes over the {2 * m // MiB} MiB-per-rank workload in 8 MiB slices shared "
                  f"round-robin by {threads} threads ({wall:.1f} s wall)",
    }


def run_copy(env: Env, steps: int, warmup: int, nbytes: int = GiB):
    snac = env.snac
    src = env.torch.randint(0, 255, (nbytes,), dtype=env.torch.uint8, device=env.dev)
    dst = env.empty(nbytes)
    t = env.time_calls(lambda: snac.snac_copy(dst, src, nbytes, env.stream), steps, warmup)
    return attach_counters(result(f"copy {nbytes // MiB} MiB", t, 2 * nbytes, nbytes), "copy")


# (threads, tile bytes, workgroups per CU, tiles in order from counters)
PROBE_SHAPES = [(64, 4096, 2, False), (64, 4096, 4, False), (64, 4096, 5, False), (64, 4096, 8, False),
                (256, 16384, 1, False), (256, 16384, 2, False), (256, 16384, 4, False),
                (64, 16384, 2, True), (256, 16384, 1, True), (256, 16384, 2, True)]


def run_ceilings(env: Env, steps: int, warmup: int, nbytes: int = GiB):
    """HBM ceilings of this machine: read-only, write-only and 1:1 copy
    streams (snac_hbm_probe) of `nbytes` each, at every launch shape of
    PROBE_SHAPES; the best shape of each kind is the ceiling."""
    snac = env.snac
    torch = env.torch
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=env.dev)
    dst = env.empty(nbytes)
    rows, best = [], {}
    for kind, moved in (("read", nbytes), ("write", nbytes), ("copy", 2 * nbytes)):
        for th, tile, w, ordered in PROBE_SHAPES:
            s = None if kind == "write" else src
            k = kind + ("_ordered" if ordered else "")
            t = env.time_calls(lambda: snac.snac_hbm_probe(k, dst, s, nbytes, th, tile, w, 0x9E3779B9,
                                                           env.stream), steps, warmup)
            gbps = moved / t / 1e9
            rows.append({"probe": kind, "threads": th, "tile_bytes": tile, "wgs_per_cu": w,
                         "tiles": "in order from counters" if ordered else "grid-stride",
                         "ms_per_call": round(t * 1e3, 5), "GBps": round(gbps, 1)})
            if gbps > best.get(kind, (0,))[0]:
                best[kind] = (gbps, th, tile, w, ordered)
    del src, dst
    torch.cuda.empty_cache()
    out = {"workload": f"HBM ceilings, {nbytes // MiB} MiB streams (snac_hbm_probe)", "shapes": rows}
    for kind, (gbps, th, tile, w, ordered) in best.items():
        out[f"{kind}_GBps"] = round(gbps, 1)
        out[f"{kind}_frac_of_peak"] = round(gbps / PEAK_GBPS, 4)
        out[f"{kind}_shape"] = (f"{th} threads, {tile} B tiles, {w} per CU, "
                                + ("tiles in order from counters" if ordered else "grid-stride tiles"))
    return out


def run_rs_ag(env: Env, steps: int, warmup: int, which=("rs", "ag", "ag_cold")):
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    rows, cols = N * 4096, 2048
    per_rank = rows * cols * 2
    src = [env.upload(gen_bf16(rows * cols, wl.CFG_RS_AG_BF16_N8, r)) for r in range(N)]
    rs_out = [env.empty(per_rank // N) for _ in range(N)]
    ag_out = [env.empty(per_rank) for _ in range(N)]
    out = []
    rs = lambda: snac.snac_reduce_scatter(env.ctx, src, rs_out, per_rank, "bf16", env.stream)
    ag = lambda: snac.snac_all_gather(env.ctx, rs_out, ag_out, per_rank // N, "bf16", env.stream)
    rs()
    if "rs" in which:
        t_rs = env.time_calls(rs, steps, warmup)
        out.append(attach_counters(result(f"reduce_scatter bf16 N={N} ({rows}x{cols})/rank", t_rs,
                                          N * per_rank + per_rank, per_rank), "rs"))
    if "ag" in which:
        t_ag = env.time_calls(ag, steps, warmup)
        ar_out = [env.empty(per_rank) for _ in range(N)]
        snac.snac_all_reduce(env.ctx, src, ar_out, per_rank, "bf16", env.stream)
        env.torch.cuda.synchronize()
        same = all(bool(env.torch.equal(a, b)) for a, b in zip(ag_out, ar_out))
        del ar_out
        out.append(attach_counters(result(f"all_gather bf16 N={N} ({rows // N}x{cols})/rank in", t_ag,
                                          per_rank + N * per_rank, per_rank,
                                          ag_of_rs_equals_allreduce=same, inputs="reused across calls"), "ag"))
    if "ag_cold" in which:
        t_ag_cold = env.time_calls_cold(ag, steps, warmup)
        out.append(attach_counters(
            result(f"all_gather bf16 N={N} ({rows // N}x{cols})/rank in, inputs evicted from the caches before "
                   "each call", t_ag_cold, per_rank + N * per_rank, per_rank, inputs="evicted before each call"),
            "ag_cold"))
    del src, rs_out, ag_out
    env.torch.cuda.empty_cache()
    return out


def run_a2a(env: Env, steps: int, warmup: int, variant: str):
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    per_rank = 128 * MiB
    e = per_rank // 4
    src = [env.upload(wl.raw_u32(e, wl.CFG_A2A_N8, r)) for r in range(N)]
    if variant == "a2a":
        dst = [env.empty(per_rank) for _ in range(N)]
        t = env.time_calls(lambda: snac.snac_all_to_all(env.ctx, src, dst, per_rank, "u32", env.stream), steps, warmup)
        return attach_counters(result(f"all_to_all u32 N={N} 128 MiB/rank", t, 2 * N * per_rank, per_rank), "a2a")
    c = wl.v_counts(N, e, N, cfg=wl.CFG_A2A_N8)
    if variant == "a2av":
        cols = c.sum(axis=0)
        dst = [env.empty(int(cols[d]) * 4) for d in range(N)]
        flat = c.reshape(-1).tolist()
        t = env.time_calls(lambda: snac.snac_all_to_all_v(env.ctx, src, dst, flat, "u32", env.stream), steps, warmup)
        return attach_counters(result(f"all_to_all_v u32 N={N} 128 MiB/rank, Dirichlet(0.5) counts", t,
                                      2 * N * per_rank, per_rank, zero_chunks=int((c == 0).sum()),
                                      unaligned_chunks=int((c % 4 != 0).sum())), "a2av")
    row = c[0].tolist()
    if variant == "agv":
        dst = [env.empty(per_rank) for _ in range(N)]
        t = env.time_calls(lambda: snac.snac_all_gather_v(env.ctx, src, dst, row, "u32", env.stream), steps, warmup)
        return attach_counters(result(f"all_gather_v u32 N={N}, counts sum 128 MiB", t, per_rank + N * per_rank,
                                      per_rank), "agv")
    dsrc = [env.upload(wl.normal_f32(e, wl.CFG_A2A_N8, r)) for r in range(N)]
    del src
    dst = [env.empty(int(row[r]) * 4) for r in range(N)]
    t = env.time_calls(lambda: snac.snac_reduce_scatter_v(env.ctx, dsrc, dst, row, "f32", env.stream), steps, warmup)
    return attach_counters(result(f"reduce_scatter_v f32 N={N}, 128 MiB/rank in", t, N * per_rank + per_rank,
                                  per_rank), "rsv")


def run_pipeline(env: Env, steps: int, warmup: int, dtype: str):
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    rows, cols = 4096, 8192
    count = rows * cols
    es = 2 if dtype == "bf16" else 4
    if dtype == "bf16":
        xs = [env.upload(gen_bf16(count, wl.CFG_PIPELINE_N8, r)) for r in range(N)]
    else:
        xs = [env.upload(wl.normal_f32(count, wl.CFG_PIPELINE_N8, r)) for r in range(N)]
    out = env.empty(count * es)
    # a staging ring that holds a whole 4096x8192 message (f32: 128 MiB) per rank
    ctx = snac.snac_init(N, 128 * MiB, env.stream)
    try:
        t = env.time_calls(lambda: snac.snac_pipeline_scale_reduce(ctx, xs, out, count, dtype, env.stream),
                           steps, warmup)
        snac.snac_check(ctx, env.stream)
    finally:
        snac.snac_finalize(ctx, env.stream)
    per_rank = count * es
    return attach_counters(result(f"snac_pipeline {dtype} N={N} ({rows}x{cols})/rank", t,
                                  3 * N * per_rank + per_rank, per_rank, staging_bytes_per_rank=128 * MiB),
                           f"pipeline_{dtype}")


def run_pipeline_latency(env: Env):
    """SNAC pipeline bf16 N=8, 1 KiB .. 1 MiB per rank: microseconds per call."""
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    top = MiB
    xs = [env.upload(gen_bf16(top // 2, wl.CFG_PIPELINE_N8, r)) for r in range(N)]
    out = env.empty(top)
    lat = {}
    for p in range(10, 21):
        b = 1 << p
        t = env.graph_median(lambda st: snac.snac_pipeline_scale_reduce(env.ctx, xs, out, b // 2, "bf16", st))
        lat[str(b)] = round(t * 1e6, 2)
    snac.snac_check(env.ctx, env.stream)
    return {"workload": f"snac_pipeline bf16 N={N} latency, bytes/rank -> us/call "
                        "(median over 20 runs of a HIP graph of 10 calls)", "us_per_call": lat}


def run_sweep_ar(env: Env, runs: int = 20, warmup: int = 5):
    return {"workload": f"allreduce bf16 N={N} sweep, 1 KiB .. 1 GiB per rank",
            "rows": sweep_rows(env, "allreduce", KiB, GiB, None, runs, warmup, 0)}


def run_sweep_ag(env: Env, runs: int = 20, warmup: int = 5):
    return {"workload": f"all_gather bf16 N={N} sweep, 128 B .. 128 MiB in per rank (1 KiB .. 1 GiB out)",
            "rows": sweep_rows(env, "all_gather", 128, 128 * MiB, None, runs, warmup, 0)}


ONLY = {
    "allreduce": lambda env, a: run_allreduce(env, a.steps, a.warmup, cpu=False, graph=False)[0],
    "allreduce_atomic": lambda env, a: run_allreduce_atomic(env, a.steps, a.warmup),
    "copy": lambda env, a: run_copy(env, a.steps, a.warmup),
    "ceilings": lambda env, a: run_ceilings(env, a.steps, a.warmup),
    "rs": lambda env, a: run_rs_ag(env, a.steps, a.warmup, ("rs",)),
    "ag": lambda env, a: run_rs_ag(env, a.steps, a.warmup, ("ag",)),
    "ag_cold": lambda env, a: run_rs_ag(env, a.steps, a.warmup, ("ag_cold",)),
    "rs_ag": lambda env, a: run_rs_ag(env, a.steps, a.warmup),
    "a2a": lambda env, a: run_a2a(env, a.steps, a.warmup, "a2a"),
    "a2av": lambda env, a: run_a2a(env, a.steps, a.warmup, "a2av"),
    "agv": lambda env, a: run_a2a(env, a.steps, a.warmup, "agv"),
    "rsv": lambda env, a: run_a2a(env, a.steps, a.warmup, "rsv"),
    "pipeline_bf16": lambda env, a: run_pipeline(env, a.steps, a.warmup, "bf16"),
    "pipeline_f32": lambda env, a: run_pipeline(env, a.steps, a.warmup, "f32"),
    "pipeline_latency": lambda env, a: run_pipeline_latency(env),
    "sweep_ar": lambda env, a: run_sweep_ar(env),
    "sweep_ag": lambda env, a: run_sweep_ag(env),
}


# ------------------------------------------------- counter summaries
# Each workload's dominant kernel (a regex on the kernel name rocprofv3
# reports), its algorithmic bytes per launch, and the source set its
# counters are tied to.
PROFILED = {
    "allreduce": (r"snac::reduce_kernel<8, snac::BF16", 2 * N * 256 * MiB, "collectives",
                  "allreduce_bf16_n8_256mib"),
    "copy": (r"snac::copy_kernel", 2 * GiB, "collectives", "copy_1gib"),
    "rs": (r"snac::reduce_kernel<8, snac::BF16", N * 128 * MiB + 128 * MiB, "collectives",
           "reduce_scatter_bf16_n8_32768x2048"),
    "ag": (r"snac::copy_kernel", 128 * MiB + N * 128 * MiB, "collectives", "all_gather_bf16_n8_4096x2048_in_reused"),
    "ag_cold": (r"snac::copy_kernel", 128 * MiB + N * 128 * MiB, "collectives",
                "all_gather_bf16_n8_4096x2048_in_evicted"),
    "a2a": (r"snac::copy_kernel", 2 * N * 128 * MiB, "collectives", "all_to_all_u32_n8_128mib"),
    "a2av": (r"snac::copy_kernel", 2 * N * 128 * MiB, "collectives", "all_to_all_v_u32_n8_128mib"),
    "agv": (r"snac::copy_kernel", 128 * MiB + N * 128 * MiB, "collectives", "all_gather_v_u32_n8_128mib"),
    "rsv": (r"snac::reduce_kernel<8, snac::F32", N * 128 * MiB + 128 * MiB, "collectives",
            "reduce_scatter_v_f32_n8_128mib"),
    "pipeline_bf16": (r"snac::pipeline_kernel<snac::BF16, 8>", 3 * N * 64 * MiB + 64 * MiB, "pipeline",
                      "snac_pipeline_bf16_n8_4096x8192"),
    "pipeline_f32": (r"snac::pipeline_kernel<snac::F32, 8>", 3 * N * 128 * MiB + 128 * MiB, "pipeline",
                     "snac_pipeline_f32_n8_4096x8192"),
}

# counter passes (one rocprofv3 --pmc run each) and what each holds
PMC_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "rdsize": ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_BUBBLE_sum"],
    "l2wr": ["TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"],
    "stall": ["TCC_EA0_WRREQ_STALL_sum", "TCC_TAG_STALL_sum", "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_WRREQ_LEVEL_sum"],
    "utcl1": ["TCP_UTCL1_TRANSLATION_MISS_sum", "TCP_UTCL1_REQUEST_sum", "TCP_PENDING_STALL_CYCLES_sum",
              "TCP_TCC_READ_REQ_LATENCY_sum"],
}


def _csv_means(dirpath: str, kernel_re: str) -> dict:
    """Mean value per counter over the dispatches of kernels matching
    kernel_re in the rocprofv3 counter CSVs under dirpath; also the kernel
    name and dispatch count."""
    import csv

    vals, name = {}, None
    for path in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if not re.search(kernel_re, r["Kernel_Name"]):
                continue
            name = r["Kernel_Name"]
            vals.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
    out = {k: sum(v.values()) / len(v) for k, v in vals.items()}
    out["_dispatches"] = max((len(v) for v in vals.values()), default=0)
    out["_kernel"] = name
    return out


def _trace_rows(dirpath: str) -> list:
    """The rows of a rocprofv3 --stats kernel summary under dirpath."""
    import csv

    rows = []
    for path in glob.glob(os.path.join(dirpath, "**", "*kernel_stats.csv"), recursive=True):
        rows.extend(csv.DictReader(open(path)))
    return rows


def _trace_stats(dirpath: str, kernel_re: str):
    """(name, calls, average ns) of the kernel matching kernel_re in a
    rocprofv3 --stats kernel summary under dirpath."""
    for r in _trace_rows(dirpath):
        if re.search(kernel_re, r["Name"]):
            return r["Name"], int(r["Calls"]), float(r["AverageNs"])
    return None


def _short(name: str) -> str:
    """A kernel name without its return type, anonymous namespaces and
    parameter list."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    return name if len(name) <= 72 else name[:69] + "..."


def trace_table(dirpath: str, top: int = 6) -> list[str]:
    rows = sorted(_trace_rows(dirpath), key=lambda r: -float(r["TotalDurationNs"]))[:top]
    out = ["| kernel | calls | average (ns) | min (ns) | max (ns) | stddev (ns) | share |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                   f"{r['MaxNs']} | {float(r['StdDev']):.0f} | {float(r['Percentage']):.2f} % |")
    return out


def summarize(workload: str, root: str, commands: list[str]) -> str:
    """A profiles/ summary (markdown) of `workload` from the rocprofv3 output
    under root/<pass>_<workload> (counter passes) and root/trace_<workload>
    (kernel trace), with the copy passes under root/<pass>_copy as the
    calibration of the FETCH_SIZE and WRITE_SIZE derived counters."""
    kre, alg, srcs, stem = PROFILED[workload]
    m = {p: _csv_means(os.path.join(root, f"{p}_{workload}"), kre) for p in PMC_PASSES}
    cal = {p: _csv_means(os.path.join(root, f"{p}_copy"), PROFILED["copy"][0]) for p in ("fetch", "write")}
    kernel = next((v["_kernel"] for v in m.values() if v.get("_kernel")), kre)
    rd, wr, l2 = m["rdsize"], m["write"], m["l2wr"]
    read_bytes = 32 * rd["TCC_EA0_RDREQ_32B_sum"] + 64 * rd["TCC_EA0_RDREQ_64B_sum"] + 128 * rd["TCC_EA0_RDREQ_128B_sum"]
    wreq, w64 = l2["TCC_EA0_WRREQ_sum"], l2["TCC_EA0_WRREQ_64B_sum"]
    write_bytes = 32 * (wreq - w64) + 64 * w64
    traffic = read_bytes + write_bytes
    hit = l2["TCC_HIT_sum"] / max(1.0, l2["TCC_HIT_sum"] + l2["TCC_MISS_sum"])
    fetch_kib, write_kib = m["fetch"]["FETCH_SIZE"], wr["WRITE_SIZE"]
    cal_fetch = GiB / (1024 * cal["fetch"]["FETCH_SIZE"])
    cal_write = GiB / (1024 * cal["write"]["WRITE_SIZE"])
    # the hash of the sources the run used, recorded on the GPU machine next to
    # its output (else the current tree's)
    hp = os.path.join(root, "source_hashes.json")
    run_hash = json.load(open(hp))[srcs] if os.path.exists(hp) else source_hash(SOURCE_SETS[srcs])
    tdir = os.path.join(root, f"trace_{workload}")
    tr = _trace_stats(tdir, kre)
    L = [f"# `bench.py --only {workload}` ({stem}): kernel trace, HBM traffic and L2 behaviour from rocprofv3", "",
         f"Dominant kernel: `{_short(kernel or kre)}`, {alg} algorithmic bytes per launch.  Every run below is "
         "its own process on the same machine, in the same session.", ""]
    if tr:
        L += ["Kernel trace (`--kernel-trace --stats`, 20 timed calls after 5 warm-up calls):", ""]
        L += trace_table(tdir) + [""]
        L += [f"Average duration of the dominant kernel: {tr[2] / 1e3:.1f} us = **{alg / tr[2]:.0f} GB/s** of "
              f"algorithmic bytes ({alg / tr[2] / PEAK_GBPS:.3f} of 8 TB/s).", ""]
        tj = os.path.join(root, f"time_{workload}.json")
        if os.path.exists(tj):
            t = json.load(open(tj))
            if isinstance(t, list):
                t = t[0]
            L += [f"Same machine, same command without the profiler (HIP events on the launch stream, "
                  f"`python3 bench.py --only {workload}`): {t['ms_per_call']} ms per call, {t['hbm_GBps']} GB/s; "
                  f"the trace's average is {100 * (tr[2] / 1e6 / t['ms_per_call'] - 1):+.1f} % from it.", ""]
    L += ["Commands, from the repository root on the GPU machine (`REPO=$PWD`; one run per pass):", ""]
    L += [f"    {c}" for c in commands] + [""]
    L += ["Bytes by request size (gfx950 has a counter per EA read size; the `FETCH_SIZE` expression counts "
          "128-byte reads through `TCC_BUBBLE`, which reads zero here, so it counts each as 64 bytes):", "",
          "| counter | per dispatch | bytes |", "|---|---|---|"]
    for k, b in (("TCC_EA0_RDREQ_32B_sum", 32), ("TCC_EA0_RDREQ_64B_sum", 64), ("TCC_EA0_RDREQ_128B_sum", 128)):
        L.append(f"| {k} | {rd[k]:.1f} | {rd[k] * b:.0f} |")
    L += [f"| TCC_BUBBLE_sum | {rd['TCC_BUBBLE_sum']:.1f} | |",
          f"| TCC_EA0_WRREQ_sum ({w64:.1f} of them 64-byte) | {wreq:.1f} | {write_bytes:.0f} |", "",
          f"Read {read_bytes:.0f} B + written {write_bytes:.0f} B = **{traffic:.0f} B per launch**, "
          f"**{traffic / alg:.5f} x** the algorithmic {alg} B.", "",
          "Derived counters, and the calibration a plain 1 GiB copy gives them (`bench.py --only copy`):", "",
          "| counter | KiB per dispatch | copy calibration (1 GiB / counter) | scaled bytes |", "|---|---|---|---|",
          f"| FETCH_SIZE | {fetch_kib:.1f} | {cal_fetch:.4f} | {fetch_kib * 1024 * cal_fetch:.0f} |",
          f"| WRITE_SIZE | {write_kib:.1f} | {cal_write:.4f} | {write_kib * 1024 * cal_write:.0f} |", "",
          f"L2 (TCC): {l2['TCC_HIT_sum']:.0f} hits, {l2['TCC_MISS_sum']:.0f} misses per dispatch, hit rate "
          f"**{hit:.3f}** (a streamed 128-byte line is one miss and one hit: two 64-byte requests).", ""]
    if m["stall"].get("_dispatches"):
        st = m["stall"]
        L += ["Stall and latency counters (sums over TCC / TCP instances, per dispatch):", "",
              "| counter | per dispatch |", "|---|---|"]
        L += [f"| {k} | {v:.0f} |" for k, v in st.items() if not k.startswith("_")]
        L += [f"| {k} | {v:.0f} |" for k, v in m["utcl1"].items() if not k.startswith("_")]
        if rd.get("TCC_EA0_RDREQ_32B_sum") is not None and st.get("TCC_EA0_RDREQ_LEVEL_sum"):
            nreq = rd["TCC_EA0_RDREQ_32B_sum"] + rd["TCC_EA0_RDREQ_64B_sum"] + rd["TCC_EA0_RDREQ_128B_sum"]
            L.append(f"| mean EA read latency: RDREQ_LEVEL / read requests (cycles) | "
                     f"{st['TCC_EA0_RDREQ_LEVEL_sum'] / max(1.0, nreq):.0f} |")
            L.append(f"| mean EA write latency: WRREQ_LEVEL / write requests (cycles) | "
                     f"{st['TCC_EA0_WRREQ_LEVEL_sum'] / max(1.0, wreq):.0f} |")
        L.append("")
    L += ["Machine-readable (read by bench.py; the hash is of the kernel sources the counters were taken with):", "",
          f"- workload: `{workload}`", f"- sources: `{srcs}`",
          f"- kernel_source_hash: `{run_hash}`",
          f"- traffic_bytes_per_launch: `{traffic:.0f}`", f"- read_bytes_per_launch: `{read_bytes:.0f}`",
          f"- write_bytes_per_launch: `{write_bytes:.0f}`", f"- algorithmic_bytes_per_launch: `{alg}`",
          f"- l2_hit: `{hit:.4f}`", f"- fetch_size_copy_calibration: `{cal_fetch:.4f}`",
          f"- write_size_copy_calibration: `{cal_write:.4f}`"]
    if tr:
        L.append(f"- kernel_average_ns: `{tr[2]:.0f}`")
    return "\n".join(L) + "\n"


def summarize_headline(root: str, commands: list[str]) -> str:
    """profiles/ summary of the headline command under the kernel trace
    (root/trace_headline), set against the default run's line from the same
    session (root/bench_line.json)."""
    line = json.load(open(os.path.join(root, "bench_line.json")))
    hp = os.path.join(root, "source_hashes.json")
    run_hash = json.load(open(hp))["collectives"] if os.path.exists(hp) else kernel_source_hash()
    tdir = os.path.join(root, "trace_headline")
    _, calls, avg = _trace_stats(tdir, PROFILED["allreduce"][0])
    alg = PROFILED["allreduce"][1]
    r = line["roofline"]
    L = ["# The headline command under rocprofv3: AllReduce bf16, N = 8, 256 MiB per rank", "",
         "The benchmark's headline path as the default run executes it, without the other workloads "
         "(`--no-extra`): 25 eager calls (5 warm-up, 20 timed with events), then 26 one-call HIP graph replays, "
         "all at 256 MiB per rank.", "", "Command (from the repository root on the GPU machine, `REPO=$PWD`):", ""]
    L += [f"    {c}" for c in commands] + [""]
    L += trace_table(tdir) + [""]
    L += [f"Average duration of `reduce_kernel<8, snac::BF16, ...>`: {avg / 1e3:.1f} us over {calls} launches = "
          f"**{alg / avg:.0f} GB/s** of algorithmic bytes (2 * 8 * 256 MiB per launch), "
          f"{alg / avg / PEAK_GBPS:.3f} of 8 TB/s.", "",
          f"Same machine, same session, `python3 bench.py` (the default run, no profiler): `ms_per_step` "
          f"{line['ms_per_step']} ms, `value` {line['value']} GB/s, `graph_median_ms` {line.get('graph_median_ms')} ms; "
          f"the trace's average kernel duration is {100 * (avg / 1e6 / line['ms_per_step'] - 1):+.1f} % from "
          "`ms_per_step`.", ""]
    if "copy_ceiling_GBps" in r:
        L += [f"Same-run ceiling (`roofline` of that line): copy {r['copy_ceiling_GBps']} GB/s; the AllReduce is at "
              f"{r['frac_of_copy_ceiling']} of it and {r['frac']} of 8 TB/s.", ""]
    L += [f"Kernel source hash (collectives): `{run_hash}`."]
    return "\n".join(L) + "\n"


def summarize_ceilings(root: str, commands: list[str]) -> str:
    """profiles/ summary of `bench.py --only ceilings` (root/ceilings.json)
    and its kernel trace (root/trace_ceilings)."""
    c = json.load(open(os.path.join(root, "ceilings.json")))
    hp = os.path.join(root, "source_hashes.json")
    run_hash = json.load(open(hp))["probes"] if os.path.exists(hp) else source_hash(SOURCE_SETS["probes"])
    L = ["# HBM ceilings of one MI355X: read-only, write-only and 1:1 copy streams of 1 GiB", "",
         "`snac_hbm_probe` streams with the collectives' access primitives (16-byte buffer loads and stores with the "
         "streaming hint) at each launch shape, the tiles grid-stride or, after 8 grid-stride rounds, in order from "
         "counters as the collectives' long launches take them; 20 timed calls after 5 warm-up calls, HIP events. "
         "Bandwidth counts the bytes each stream must move (copy: read + written).", "",
         "Commands (from the repository root on the GPU machine, `REPO=$PWD`):", "",
         "    python3 $REPO/bench.py --only ceilings"]
    L += [f"    {x}" for x in commands] + ["",
          "| probe | threads | tile (B) | WGs per CU | tiles | ms per call | GB/s |", "|---|---|---|---|---|---|---|"]
    for r in c["shapes"]:
        L.append(f"| {r['probe']} | {r['threads']} | {r['tile_bytes']} | {r['wgs_per_cu']} | "
                 f"{r.get('tiles', 'grid-stride')} | {r['ms_per_call']} | {r['GBps']} |")
    L += ["", "Best shape of each kind (the ceiling on this machine):", "", "| stream | GB/s | of 8 TB/s | shape |",
          "|---|---|---|---|"]
    for k in ("read", "write", "copy"):
        L.append(f"| {k} | {c[k + '_GBps']} | {c[k + '_frac_of_peak']} | {c[k + '_shape']} |")
    L += ["", "Kernel trace of the same command under the profiler (probe_kernel<kind, threads, tile>; "
          "kind 0 read, 1 write, 2 copy):", ""]
    L += trace_table(os.path.join(root, "trace_ceilings"), top=24) + ["", f"Kernel source hash (probes): `{run_hash}`."]
    return "\n".join(L) + "\n"


def rows_of(item):
    """The JSONL rows of one result (sweeps expand into their sizes)."""
    if isinstance(item, list):
        out = []
        for x in item:
            out.extend(rows_of(x))
        return out
    if isinstance(item, dict) and "rows" in item:
        return list(item["rows"])
    return [item]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default=None, choices=sorted(ONLY))
    ap.add_argument("--coll", default=None, help="per-collective sweep: NAME then the pages' positional arguments")
    ap.add_argument("pos", nargs="*", help="[minBytes [maxBytes [graphLaunches [runs [warmup [seed]]]]]] for --coll")
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--nranks", type=int, default=N)
    ap.add_argument("--jsonl", default=None, help="append one JSON line per measured row to this file")
    ap.add_argument("--sweep", action="store_true", help="same as --coll allreduce 1K 1G")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--summarize", default=None, metavar="WORKLOAD",
                    help="write the profiles/ summary of WORKLOAD (a --only name, 'headline' or 'ceilings') from "
                         "the rocprofv3 output under --prof-dir")
    ap.add_argument("--prof-dir", default=os.path.join(ROOT, "rocprof_out"))
    ap.add_argument("--commands", default=None, help="file listing the rocprofv3 commands that made --prof-dir")
    args = ap.parse_args()
    if args.summarize:
        cmds = open(args.commands).read().splitlines() if args.commands else []
        cmds = [c for c in cmds if c.strip()]
        if args.summarize == "headline":
            text = summarize_headline(args.prof_dir, cmds)
            dest = os.path.join(PROFILES, "allreduce_bf16_n8_256mib_headline_kernel_trace.md")
        elif args.summarize == "ceilings":
            text = summarize_ceilings(args.prof_dir, cmds)
            dest = os.path.join(PROFILES, "hbm_ceilings_1gib.md")
        else:
            text = summarize(args.summarize, args.prof_dir, cmds)
            dest = os.path.join(PROFILES, f"{PROFILED[args.summarize][3]}_counters.md")
        with open(dest, "w", encoding="utf-8") as f:
            f.write(text)
        print(dest)
        return 0
    if args.gpus != 1:
        print(f"bench.py: the library runs its N logical ranks in one GPU's HBM; --gpus {args.gpus} "
              "is not supported (nothing here uses a second GPU)", file=sys.stderr)
        return 2
    if args.pos and not args.coll:
        ap.error("positional size arguments go with --coll")
    global COUNTERS
    COUNTERS = read_counter_summaries()
    jsonl = open(args.jsonl, "a") if args.jsonl else None
    env = Env()
    if args.sweep and not args.coll:
        args.coll, args.pos = "allreduce", ["1K", "1G"]
    if args.coll:
        coll = ALIASES.get(args.coll, ALIASES.get(args.coll.upper(), args.coll))
        if coll not in SPECS:
            raise SystemExit(f"unknown collective {args.coll}: one of {', '.join(SPECS)}")
        p = args.pos + [None] * (6 - len(args.pos))
        lo = parse_size(p[0]) if p[0] else KiB
        hi = parse_size(p[1]) if p[1] else lo
        graph_launches = int(p[2]) if p[2] else 10
        runs = int(p[3]) if p[3] else 20
        warmup = int(p[4]) if p[4] else 5
        seed = int(p[5]) if p[5] else 0
        sweep_rows(env, coll, lo, hi, graph_launches, runs, warmup, seed, dtype=args.dtype, n=args.nranks,
                   jsonl=jsonl, emit=True)
        env.snac.snac_finalize(env.ctx, env.stream)
        return 0
    if args.only:
        r = ONLY[args.only](env, args)
        print(json.dumps(r), flush=True)
        if jsonl:
            for x in rows_of(r):
                jsonl.write(json.dumps(x) + "\n")
        env.snac.snac_finalize(env.ctx, env.stream)
        return 0

    head, cpu = run_allreduce(env, args.steps, args.warmup, cpu=not args.no_cpu)
    extra = []
    ceilings = None
    if not args.no_extra:
        env.torch.cuda.empty_cache()
        extra.append(run_copy(env, args.steps, args.warmup))
        ceilings = run_ceilings(env, args.steps, args.warmup)
        extra.append(ceilings)
        extra.extend(run_rs_ag(env, args.steps, args.warmup))
        for v in ("a2a", "a2av", "agv", "rsv"):
            extra.append(run_a2a(env, args.steps, args.warmup, v))
            env.torch.cuda.empty_cache()
        for dt in ("bf16", "f32"):
            extra.append(run_pipeline(env, args.steps, args.warmup, dt))
        extra.append(run_pipeline_latency(env))
        env.torch.cuda.empty_cache()
        extra.append(run_allreduce_atomic(env, 3, 1))
        env.torch.cuda.empty_cache()
        extra.append(run_sweep_ar(env))
        extra.append(run_sweep_ag(env))
    achieved = head["hbm_GBps"]
    roofline = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4),
        "traffic": head.get("traffic_bytes"),
    }
    if ceilings:
        copy_ceiling = max(ceilings.get("copy_GBps", 0.0), extra[0]["hbm_GBps"])
        roofline["copy_ceiling_GBps"] = round(copy_ceiling, 1)
        roofline["frac_of_copy_ceiling"] = round(achieved / copy_ceiling, 4)
    line = {
        "metric": METRIC,
        "value": achieved,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "nranks": N,
            "bytes_per_rank": 256 * MiB,
            "parallelism": "one GPU, 8 logical ranks in its HBM",
        },
        "algbw_GBps": head["algbw_GBps"],
        "graph_median_ms": head.get("graph_median_ms"),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    if jsonl:
        for x in [head] + rows_of(extra):
            jsonl.write(json.dumps(x) + "\n")
    env.snac.snac_finalize(env.ctx, env.stream)
    return 0


if __name__ == "__main__":
    sys.exit(main())
