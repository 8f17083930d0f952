"""bench.py's measurement plumbing on the CPU: size arguments in the pages'
form, and the counter summaries -- bytes counted from EA requests by size,
the copy calibration of the derived counters, L2 hit rate, the kernel trace
and the same-machine timing -- built from synthetic rocprofv3 output with known
values, then read back by the benchmark as current or stale."""
from __future__ import annotations

import csv
import json
import os

import pytest

import bench

GiB = 1 << 30


def test_parse_size():
    assert bench.parse_size("1K") == 1024
    assert bench.parse_size("128M") == 128 << 20
    assert bench.parse_size("1G") == GiB
    assert bench.parse_size("4096") == 4096
    assert bench.parse_size("64KiB") == 64 << 10
    with pytest.raises(SystemExit):
        bench.parse_size("12X")


def _counters(path, kernel, values, dispatches=(1, 2, 3)):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d in dispatches:
            for name, v in values.items():
                # the value varies by dispatch; the summary uses the mean
                w.writerow({"Dispatch_Id": d, "Kernel_Name": kernel, "Counter_Name": name,
                            "Counter_Value": v * (1 + (d - 2) * 0.01)})
        w.writerow({"Dispatch_Id": 99, "Kernel_Name": "other_kernel()", "Counter_Name": next(iter(values)),
                    "Counter_Value": 1e12})


def _stats(path, kernel, avg_ns):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_kernel_stats.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                          "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": kernel, "Calls": 25, "TotalDurationNs": 25 * avg_ns, "AverageNs": avg_ns,
                    "Percentage": 99.9, "MinNs": avg_ns - 10, "MaxNs": avg_ns + 10, "StdDev": 5})


def test_summary_counts_bytes_by_request_size(tmp_path, monkeypatch):
    root = str(tmp_path / "prof")
    kern = "void snac::reduce_kernel<8, snac::BF16, 1, true, false>(snac_coll_desc)"
    copyk = "void snac::copy_kernel<1, true, 64, 4096u>(snac_coll_desc)"
    # AllReduce, 256 MiB per rank: 2 GiB read as 128-byte requests plus a few
    # 64- and 32-byte ones; 2 GiB written as 64-byte requests plus 32-byte ones
    r128, r64, r32 = 16777216, 1000, 10
    w_all, w64 = 33554432 + 20, 33554432
    _counters(f"{root}/rdsize_allreduce", kern, {"TCC_EA0_RDREQ_32B_sum": r32, "TCC_EA0_RDREQ_64B_sum": r64,
                                                 "TCC_EA0_RDREQ_128B_sum": r128, "TCC_BUBBLE_sum": 0})
    _counters(f"{root}/l2wr_allreduce", kern, {"TCC_HIT_sum": 1000, "TCC_MISS_sum": 3000,
                                               "TCC_EA0_WRREQ_sum": w_all, "TCC_EA0_WRREQ_64B_sum": w64})
    _counters(f"{root}/fetch_allreduce", kern, {"FETCH_SIZE": 1048576})
    _counters(f"{root}/write_allreduce", kern, {"WRITE_SIZE": 2097152})
    _counters(f"{root}/fetch_copy", copyk, {"FETCH_SIZE": 524288})
    _counters(f"{root}/write_copy", copyk, {"WRITE_SIZE": 1048576})
    _stats(f"{root}/trace_allreduce", kern, 760000.0)
    with open(f"{root}/time_allreduce.json", "w") as f:
        json.dump({"ms_per_call": 0.76, "hbm_GBps": 5651.3}, f)
    with open(f"{root}/source_hashes.json", "w") as f:
        json.dump({"collectives": "feedfacecafebeef", "pipeline": "x", "probes": "y"}, f)
    text = bench.summarize("allreduce", root, ["rocprofv3 --pmc ... -- python3 bench.py --only allreduce"])
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": `" in line:
            k, v = line[2:].split(": `", 1)
            vals[k] = v.rstrip("`")
    read = 32 * r32 + 64 * r64 + 128 * r128
    write = 32 * (w_all - w64) + 64 * w64
    assert int(vals["read_bytes_per_launch"]) == read
    assert int(vals["write_bytes_per_launch"]) == write
    assert int(vals["traffic_bytes_per_launch"]) == read + write
    assert int(vals["algorithmic_bytes_per_launch"]) == 2 * 8 * 256 * (1 << 20)
    assert float(vals["l2_hit"]) == pytest.approx(0.25, abs=1e-4)
    assert float(vals["fetch_size_copy_calibration"]) == pytest.approx(2.0, abs=1e-4)
    assert float(vals["write_size_copy_calibration"]) == pytest.approx(1.0, abs=1e-4)
    assert vals["kernel_source_hash"] == "feedfacecafebeef"  # recorded on the GPU machine, not this tree's
    assert int(vals["kernel_average_ns"]) == 760000
    assert "+0.0 % from it" in text  # the trace's average against the same-machine event timing
    assert "other_kernel" not in text

    # read back by the benchmark: stale (hash of another tree), then current
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "allreduce_counters.md").write_text(text)
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.read_counter_summaries() == {}
    (prof / "allreduce_counters.md").write_text(text.replace("feedfacecafebeef", bench.kernel_source_hash()))
    got = bench.read_counter_summaries()
    assert set(got) == {"allreduce"} and int(got["allreduce"]["traffic_bytes_per_launch"]) == read + write
    monkeypatch.setattr(bench, "COUNTERS", got)
    row = bench.attach_counters({"algorithmic_bytes": 2 * 8 * 256 * (1 << 20)}, "allreduce")
    assert row["traffic_over_algorithmic"] == pytest.approx((read + write) / (2 * 8 * 256 * (1 << 20)), abs=1e-5)
    assert row["l2_hit"] == pytest.approx(0.25, abs=1e-4)
    assert bench.attach_counters({}, "copy")["traffic_bytes"] is None


def test_kernel_names_are_shortened_for_tables():
    assert bench._short("void snac::(anonymous namespace)::probe_kernel<0, 64, 4096u>(char*, char const*, "
                        "unsigned long, unsigned int)") == "snac::probe_kernel<0, 64, 4096u>"
    assert bench._short("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
