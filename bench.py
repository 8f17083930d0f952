"""Benchmark of the copy / N-to-1 reduce collective datapath on one MI355X.

Default run (the headline): AllReduce(sum) over N = 8 logical ranks, bf16
inputs with binary32 accumulation and bf16 output, 256 MiB per rank, the
result written to all 8 destination buffers.  A step is one AllReduce call
(one kernel) over inputs already resident in HBM.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Prints one JSON line.  ``value`` is the algorithmic HBM bandwidth of the
AllReduce, 2 * N * B bytes per call (every source read once, every
destination written once) over the measured time per call.  ``roofline``
relates that to the 8 TB/s HBM peak; ``traffic`` is the HBM traffic per
launch from rocprofv3 counters when the recorded counters match the current
kernel sources (else null).  ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.  ``extra`` holds the other configured
collectives (ReduceScatter then AllGather, AllToAll / AllToAllV, AllGatherV,
ReduceScatterV, the SNAC pipeline, and a plain copy) measured the same way.

Other modes:
    --only NAME     run one workload (allreduce, allreduce_atomic, copy, rs_ag,
                    a2a, a2av, agv, rsv, pipeline_bf16, pipeline_f32,
                    pipeline_latency) --
                    for profiler runs
    --sweep         AllReduce bf16 N=8 over 1 KiB .. 1 GiB per rank (JSON
                    lines to stdout; small sizes batched in a HIP graph)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s & % of peak, 8-logical-rank bf16 AllReduce reduceN, 256 MiB/rank"
PEAK_GBPS = 8000.0
MiB = 1 << 20
GiB = 1 << 30
N = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "allreduce_bf16_n8_256mib_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources of the collective kernel (the dominant kernel of the benchmark)
KERNEL_SOURCES = ("include/snac_device.hpp", "include/snac_layout.hpp", "include/snac.h",
                  "copy_reduce_snac_amd/csrc/collectives.hip", "copy_reduce_snac_amd/csrc/internal.hpp")


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


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic() -> float | None:
    """HBM bytes per AllReduce launch from the counter summary, if it was
    taken with the current kernel sources."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in txt.splitlines():
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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
        return self.torch.empty(nbytes, dtype=self.torch.uint8, device=self.dev)

    def time_calls(self, fn, steps: int, warmup: int) -> float:
        """Seconds per call: events on the launch stream around `steps` calls."""
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


def gen_bf16(m: int, cfg: int, rank: int) -> np.ndarray:
    from copy_reduce_snac_amd import workloads as wl

    return wl.normal_bf16(m, cfg, rank)


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


# ------------------------------------------------------------------ workloads
def run_allreduce(env: Env, steps: int, warmup: int, per_rank: int = 256 * MiB, cpu: bool = True):
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    m = per_rank // 2
    t0 = time.time()
    host = [gen_bf16(m, wl.CFG_AR_BF16_N8, r) for r in range(N)]
    src = [env.upload(h) for h in host]
    dst = [env.empty(per_rank) for _ in range(N)]
    log(f"allreduce: inputs ready in {time.time() - t0:.1f}s")

    def call():
        snac.snac_all_reduce(env.ctx, src, dst, per_rank, "bf16", env.stream)

    t = env.time_calls(call, steps, warmup)
    alg = 2 * N * per_rank
    out = result(f"allreduce_sum bf16 N={N} {per_rank // MiB} MiB/rank", t, alg, per_rank)
    cpu_res = None
    if cpu:
        cpu_res = cpu_baseline_allreduce(host, dst, per_rank)
    return out, cpu_res


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
    got = dst[0].cpu().numpy().view(np.uint16)
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
    return {
        "value": round(value, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole 256 MiB-per-rank workload in 32 MiB slices, cycled {done / m:.1f} times "
                  f"(NumPy, single thread, {spent:.1f} s); GPU output equal on the first pass: {ok}",
        "host_cpu": platform.processor() or platform.machine(),
        "host_threads_available": len(os.sched_getaffinity(0)),
        "parallel": cpu_baseline_allreduce_threads(host, m),
    }


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
    return result(f"copy {nbytes // MiB} MiB", t, 2 * nbytes, nbytes)


def run_rs_ag(env: Env, steps: int, warmup: int):
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    rows, cols = N * 4096, 2048
    per_rank = rows * cols * 2
    src = [env.upload(gen_bf16(rows * cols, wl.CFG_RS_AG_BF16_N8, r)) for r in range(N)]
    rs_out = [env.empty(per_rank // N) for _ in range(N)]
    ag_out = [env.empty(per_rank) for _ in range(N)]
    t_rs = env.time_calls(lambda: snac.snac_reduce_scatter(env.ctx, src, rs_out, per_rank, "bf16", env.stream),
                          steps, warmup)
    ag = lambda: snac.snac_all_gather(env.ctx, rs_out, ag_out, per_rank // N, "bf16", env.stream)
    t_ag = env.time_calls(ag, steps, warmup)
    t_ag_cold = env.time_calls_cold(ag, steps, warmup)
    ar_out = [env.empty(per_rank) for _ in range(N)]
    snac.snac_all_reduce(env.ctx, src, ar_out, per_rank, "bf16", env.stream)
    env.torch.cuda.synchronize()
    same = all(bool(env.torch.equal(a, b)) for a, b in zip(ag_out, ar_out))
    return [
        result(f"reduce_scatter bf16 N={N} ({rows}x{cols})/rank", t_rs, N * per_rank + per_rank, per_rank),
        result(f"all_gather bf16 N={N} ({rows // N}x{cols})/rank in", t_ag, per_rank + N * per_rank, per_rank,
               ag_of_rs_equals_allreduce=same),
        result(f"all_gather bf16 N={N} ({rows // N}x{cols})/rank in, inputs evicted from the caches before each call",
               t_ag_cold, per_rank + N * per_rank, per_rank),
    ]


def run_a2a(env: Env, steps: int, warmup: int, variant: str):
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    per_rank = 128 * MiB
    e = per_rank // 4
    src = [env.upload(wl.raw_u32(e, wl.CFG_A2A_N8, r)) for r in range(N)]
    if variant == "a2a":
        dst = [env.empty(per_rank) for _ in range(N)]
        t = env.time_calls(lambda: snac.snac_all_to_all(env.ctx, src, dst, per_rank, "u32", env.stream), steps, warmup)
        return result(f"all_to_all u32 N={N} 128 MiB/rank", t, 2 * N * per_rank, per_rank)
    c = wl.v_counts(N, e, N, cfg=wl.CFG_A2A_N8)
    if variant == "a2av":
        cols = c.sum(axis=0)
        dst = [env.empty(int(cols[d]) * 4) for d in range(N)]
        flat = c.reshape(-1).tolist()
        t = env.time_calls(lambda: snac.snac_all_to_all_v(env.ctx, src, dst, flat, "u32", env.stream), steps, warmup)
        return result(f"all_to_all_v u32 N={N} 128 MiB/rank, Dirichlet(0.5) counts", t, 2 * N * per_rank, per_rank,
                      zero_chunks=int((c == 0).sum()), unaligned_chunks=int((c % 4 != 0).sum()))
    row = c[0].tolist()
    if variant == "agv":
        dst = [env.empty(per_rank) for _ in range(N)]
        t = env.time_calls(lambda: snac.snac_all_gather_v(env.ctx, src, dst, row, "u32", env.stream), steps, warmup)
        return result(f"all_gather_v u32 N={N}, counts sum 128 MiB", t, per_rank + N * per_rank, per_rank)
    dsrc = [env.upload(wl.normal_f32(e, wl.CFG_A2A_N8, r)) for r in range(N)]
    dst = [env.empty(int(row[r]) * 4) for r in range(N)]
    t = env.time_calls(lambda: snac.snac_reduce_scatter_v(env.ctx, dsrc, dst, row, "f32", env.stream), steps, warmup)
    return result(f"reduce_scatter_v f32 N={N}, 128 MiB/rank in", t, N * per_rank + per_rank, per_rank)


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
    return result(f"snac_pipeline {dtype} N={N} ({rows}x{cols})/rank", t, 3 * N * per_rank + per_rank, per_rank,
                  staging_bytes_per_rank=128 * MiB)


def graph_time(env: Env, call, batch: int = 10, reps: int = 20) -> float:
    """Median seconds per call: `batch` calls captured in one HIP graph,
    replayed `reps` times, each replay timed with events."""
    torch = env.torch
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call(torch.cuda.current_stream())  # first launch outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(batch):
                call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3 / batch)
    return float(np.median(times))


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
        t = graph_time(env, lambda st: snac.snac_pipeline_scale_reduce(env.ctx, xs, out, b // 2, "bf16", st))
        lat[str(b)] = round(t * 1e6, 2)
    snac.snac_check(env.ctx, env.stream)
    return {"workload": f"snac_pipeline bf16 N={N} latency, bytes/rank -> us/call (HIP graph, 10 calls)",
            "us_per_call": lat}


def run_sweep(env: Env):
    """AllReduce bf16 N=8, per-rank 1 KiB .. 1 GiB; below 64 MiB the calls
    are captured 10 at a time in a HIP graph and the graph is replayed."""
    from copy_reduce_snac_amd import workloads as wl

    snac = env.snac
    top = GiB
    src = [env.upload(gen_bf16(top // 2, wl.CFG_AR_BF16_N8, r)) for r in range(N)]
    dst = [env.empty(top) for _ in range(N)]
    p = 10
    while (1 << p) <= top:
        b = 1 << p
        if b < 64 * MiB:
            t = graph_time(env, lambda st: snac.snac_all_reduce(env.ctx, src, dst, b, "bf16", st))
        else:
            t = env.time_calls(lambda: snac.snac_all_reduce(env.ctx, src, dst, b, "bf16", env.stream), 10, 3)
        r = result(f"allreduce_sum bf16 N={N} {b} B/rank", t, 2 * N * b, b,
                   cache_resident=bool(2 * N * b < 256 * MiB))
        print(json.dumps(r), flush=True)
        p += 1


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default=None)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs its N logical ranks in one GPU's HBM; --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        return 2
    env = Env()
    if args.sweep:
        run_sweep(env)
        return 0
    if args.only:
        name = args.only
        if name == "allreduce":
            r, _ = run_allreduce(env, args.steps, args.warmup, cpu=False)
        elif name == "allreduce_atomic":
            r = run_allreduce_atomic(env, args.steps, args.warmup)
        elif name == "copy":
            r = run_copy(env, args.steps, args.warmup)
        elif name == "rs_ag":
            r = run_rs_ag(env, args.steps, args.warmup)
        elif name in ("a2a", "a2av", "agv", "rsv"):
            r = run_a2a(env, args.steps, args.warmup, name)
        elif name == "pipeline_latency":
            r = run_pipeline_latency(env)
        elif name.startswith("pipeline_"):
            r = run_pipeline(env, args.steps, args.warmup, name.split("_", 1)[1])
        else:
            raise SystemExit(f"unknown workload {name}")
        print(json.dumps(r), flush=True)
        return 0

    head, cpu = run_allreduce(env, args.steps, args.warmup, cpu=not args.no_cpu)
    extra = []
    if not args.no_extra:
        env.torch.cuda.empty_cache()
        extra.append(run_copy(env, args.steps, args.warmup))
        extra.extend(run_rs_ag(env, args.steps, args.warmup))
        for v in ("a2a", "a2av", "agv", "rsv"):
            extra.append(run_a2a(env, args.steps, args.warmup, v))
            env.torch.cuda.empty_cache()
        for dt in ("bf16", "f32"):
            extra.append(run_pipeline(env, args.steps, args.warmup, dt))
        extra.append(run_pipeline_latency(env))
        env.torch.cuda.empty_cache()
        extra.append(run_allreduce_atomic(env, 3, 1))
    t = head["ms_per_call"] / 1e3
    achieved = head["hbm_GBps"]
    traffic = recorded_traffic()
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
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    env.snac.snac_finalize(env.ctx, env.stream)
    return 0


if __name__ == "__main__":
    sys.exit(main())
