"""Measure launch parameters per collective and size on the GPU at hand and
install them as tuning rules (snac_set_tuning_rules, include/snac.h).

    python -m copy_reduce_snac_amd.autotune [--out rules.json] [--sizes 64K,1M,16M,256M]
                                            [--steps 10] [--quick]

For each workload (AllReduce bf16, ReduceScatter bf16, AllGather u32,
AllToAll u32, copy; N = 8) and each per-rank size, every candidate
(workgroups per CU x cache policy) is timed with HIP events over `steps`
calls on synthetic buffers, after checking that it gives the same bytes as
the library default.  The fastest candidate per (workload, size) becomes a
rule covering the sizes from halfway (geometrically) to the next smaller
measured size up to halfway to the next larger one.  The rules are printed
as JSON, written to --out, and installed in this process; load them into
another process with snac_set_tuning_rules(json.load(...)).

Measurements on MI355X vary from machine to machine by up to 13 % in absolute HBM
bandwidth, so a table is best measured on the machine that will use it.
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import copy_reduce_snac_amd as snac

WPC = (1, 2, 4)
POLICIES = (1, 2, 3, 4)  # streaming, streaming stores, streaming loads, cached
N = 8


def _parse_size(s: str) -> int:
    m = {"K": 1 << 10, "M": 1 << 20, "G": 1 << 30}
    return int(s[:-1]) * m[s[-1]] if s[-1] in m else int(s)


def _workloads(torch, dev, per_rank: int, ctx: int):
    """name -> (rule coll, esize (0: any), per-rank input bytes, call(), output tensors)."""
    u8 = torch.uint8
    srcs = [torch.randint(0, 255, (per_rank,), dtype=u8, device=dev) for _ in range(N)]
    for s in srcs:  # finite bf16 / f32 values: clear the exponent's top bit of every 16-bit word
        s.view(torch.int16).bitwise_and_(0x3FFF)
    out = {}
    ar = [torch.empty(per_rank, dtype=u8, device=dev) for _ in range(N)]
    out["allreduce_bf16"] = (snac.SNAC_COLL_ALL_REDUCE, 2, per_rank,
                             lambda: snac.snac_all_reduce(ctx, srcs, ar, per_rank, "bf16"), ar)
    if per_rank % (N * 2) == 0:
        rs = [torch.empty(per_rank // N, dtype=u8, device=dev) for _ in range(N)]
        out["reduce_scatter_bf16"] = (snac.SNAC_COLL_REDUCE_SCATTER, 2, per_rank,
                                      lambda: snac.snac_reduce_scatter(ctx, srcs, rs, per_rank, "bf16"), rs)
    ag_in = per_rank // N
    if ag_in % 4 == 0 and ag_in:
        ag = [torch.empty(ag_in * N, dtype=u8, device=dev) for _ in range(N)]
        out["all_gather_u32"] = (snac.SNAC_COLL_ALL_GATHER, 0, ag_in,
                                 lambda: snac.snac_all_gather(ctx, srcs, ag, ag_in, "u32"), ag)
    if per_rank % (N * 4) == 0:
        a2a = [torch.empty(per_rank, dtype=u8, device=dev) for _ in range(N)]
        out["all_to_all_u32"] = (snac.SNAC_COLL_ALL_TO_ALL, 0, per_rank,
                                 lambda: snac.snac_all_to_all(ctx, srcs, a2a, per_rank, "u32"), a2a)
    cp = torch.empty(per_rank, dtype=u8, device=dev)
    out["copy"] = (snac.SNAC_RULE_ATOM_COPY, 0, per_rank, lambda: snac.snac_copy(cp, srcs[0], per_rank), [cp])
    return out, srcs


def _time(torch, fn, steps: int) -> float:
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure(sizes, steps: int = 10, log=print) -> list[dict]:
    import torch

    dev = torch.device("cuda:0")
    ctx = snac.snac_init(N, 0)
    best: dict[str, list[tuple[int, int, int, float]]] = {}
    meta = {}
    saved = snac.snac_get_tuning()
    try:
        for size in sizes:
            wl, _ = _workloads(torch, dev, size, ctx)
            for name, (coll, esize, nbytes, call, outs) in wl.items():
                meta[name] = (coll, esize)
                snac.snac_set_tuning(wgs_per_cu=0, cache_policy=0)
                default_ms = _time(torch, call, steps)
                ref = [o.clone() for o in outs]
                results = []
                for w in WPC:
                    for cp in POLICIES:
                        snac.snac_set_tuning(wgs_per_cu=w, cache_policy=cp)
                        ms = _time(torch, call, steps)
                        if not all(bool(torch.equal(o, r)) for o, r in zip(outs, ref)):
                            raise RuntimeError(f"{name} {size} wpc={w} cp={cp}: output differs from the default's")
                        results.append((ms, w, cp))
                ms, w, cp = min(results)
                log(json.dumps({"workload": name, "bytes_per_rank": nbytes, "best_ms": round(ms, 5),
                                "default_ms": round(default_ms, 5), "wgs_per_cu": w, "cache_policy": cp}))
                best.setdefault(name, []).append((nbytes, w, cp, ms))
    finally:
        snac.snac_set_tuning(**saved)
        snac.snac_finalize(ctx)
    rules = []
    for name, rows in best.items():
        coll, esize = meta[name]
        rows.sort()
        for i, (size, w, cp, _) in enumerate(rows):
            lo = 0 if i == 0 else int(math.sqrt(rows[i - 1][0] * size)) + 1
            hi = 2 ** 64 - 1 if i == len(rows) - 1 else int(math.sqrt(size * rows[i + 1][0]))
            ranks = 1 if coll == snac.SNAC_RULE_ATOM_COPY else N  # snac_copy calls have one source
            rules.append({"coll": coll, "min_ranks": ranks, "max_ranks": ranks, "esize": esize,
                          "min_bytes": lo, "max_bytes": hi, "wgs_per_cu": w, "cache_policy": cp})
    # everything the table does not name keeps the built-in behaviour
    rules.extend(snac_builtin_rules())
    return rules


def snac_builtin_rules() -> list[dict]:
    cur = snac.snac_get_tuning_rules()
    snac.snac_set_tuning_rules(None)
    try:
        return snac.snac_get_tuning_rules()
    finally:
        snac.snac_set_tuning_rules(cur)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--sizes", default="64K,1M,16M,64M,256M")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    sizes = [_parse_size(s) for s in args.sizes.split(",")]
    rules = measure(sizes, args.steps, log=lambda s: print(s, file=sys.stderr, flush=True))
    snac.snac_set_tuning_rules(rules)
    txt = json.dumps(rules, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(txt + "\n")
    print(txt)
    return 0


if __name__ == "__main__":
    sys.exit(main())
