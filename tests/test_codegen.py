"""Properties of the gfx950 code the compiler emits for the kernels
(CPU only: hipcc cross-compiles to assembly, nothing runs).

* In the SNAC pipeline kernel every workgroup barrier must sit in the
  ticket loop itself, never inside a nested loop.  When the compiler
  cannot prove the loop's control flow uniform it may split the loop so
  that the lanes of one wave reach a barrier on different iterations,
  which deadlocks the workgroup.
* No packed fp32 arithmetic (the build disables that target feature).
* No writes through the scalar data cache: no scalar memory stores or
  atomics and no scalar cache write-back or discard, in any kernel; data
  leaves the kernels through vector stores only.
* A copy tile whose source is not dword-aligned issues all its loads
  (dwordx4 and the extra dword of each unit) before waiting on any of
  them.  With a branch inside each unit's load the compiler had waited for
  every unit in turn, one load group in flight per wave.
* Full byte-misaligned tiles of the 256-thread copy kernels take the next
  lane's bytes through DPP whole-wave shifts (wave_shl:1).
* The shared tile counter's fetch in the 16 KiB-tile kernels is a plain
  global atomic that stays in flight: no wave-wide reduction around it
  (v_mbcnt) and no wait for every memory operation right after it (the
  build turns the compiler's atomic optimizer off for this), and nothing
  spills to scratch.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "copy_reduce_snac_amd", "csrc")

hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
pytestmark = pytest.mark.skipif(hipcc is None, reason="hipcc not available")

PACKED = ["v_pk_" + op + "_f32" for op in ("add", "mul", "fma")]


SOURCES = {
    "collectives.hip": os.path.join(CSRC, "collectives.hip"),
    "probes.hip": os.path.join(CSRC, "probes.hip"),
    "pipeline.hip": os.path.join(CSRC, "pipeline.hip"),
    "devapi_kernels.hip": os.path.join(ROOT, "tests", "devapi", "devapi_kernels.hip"),
}
@pytest.fixture(scope="module")
def asm(tmp_path_factory) -> dict[str, str]:
    """gfx950 assembly of every source, the compiles run side by side."""
    from copy_reduce_snac_amd.build import DEVICE_FLAGS, SOURCE_FLAGS

    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in DEVICE_FLAGS if f not in ("-fPIC",)]
    procs = {}
    for name, path in SOURCES.items():
        out = d / (name + ".s")
        cmd = [hipcc, *flags, *SOURCE_FLAGS.get(name, []), "--cuda-device-only", "-S", path, "-o", str(out)]
        procs[name] = (out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE))
    res = {}
    for name, (out, p) in procs.items():
        _, err = p.communicate()
        assert p.returncode == 0, f"{name}: {err.decode()[-2000:]}"
        res[name] = out.read_text()
    return res


def _kernels(asm: str) -> dict[str, list[str]]:
    out = {}
    cur = None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):\s", line + " ")
        if m and not line.startswith("\t"):
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is not None:
            out[cur].append(line)
            if "s_endpgm" in line:
                cur = None
    return out


def _barrier_depths(lines: list[str]) -> list[int]:
    depth = 0
    found = []
    for l in lines:
        m = re.match(r"^\.LBB\d+_\d+:(.*)", l)
        if m:
            d = re.search(r"Depth=(\d+)", m.group(1))
            depth = int(d.group(1)) if d else 0
        if "s_barrier" in l:
            found.append(depth)
    return found


def test_pipeline_barriers_only_in_the_ticket_loop(asm):
    ks = {k: v for k, v in _kernels(asm["pipeline.hip"]).items() if "pipeline_kernel" in k}
    assert len(ks) == 32
    for name, lines in ks.items():
        depths = _barrier_depths(lines)
        assert depths, name
        assert max(depths) <= 1, f"{name}: barrier inside a nested loop"


@pytest.mark.parametrize("src", sorted(SOURCES))
def test_no_packed_fp32(asm, src):
    for op in PACKED:
        assert op not in asm[src], f"{src}: {op} emitted"


SCALAR_WRITES = re.compile(r"^\s*(s_store_|s_buffer_store_|s_scratch_store_|s_atomic_|s_buffer_atomic_|"
                           r"s_dcache_wb|s_dcache_discard)", re.M)


@pytest.mark.parametrize("src", sorted(SOURCES))
def test_no_scalar_cache_writes(asm, src):
    bad = SCALAR_WRITES.findall(asm[src])
    assert not bad, f"{src}: {sorted(set(bad))}"


def _longest_unwaited_run(lines: list[str], op: str) -> int:
    """Most `op` instructions issued in a row with no s_waitcnt on vector
    memory between them."""
    best = run = 0
    for l in lines:
        t = l.strip()
        if t.startswith(op + " "):
            run += 1
            best = max(best, run)
        elif t.startswith("s_waitcnt") and "vmcnt" in t:
            run = 0
    return best


@pytest.mark.parametrize("shape", ["Li64ELj4096E", "Li256ELj16384E", "Li64ELj16384E"])
def test_misaligned_copy_tile_issues_every_load_first(asm, shape):
    # generic (not aligned) copy kernels of each tile shape, every cache policy
    ks = {k: v for k, v in _kernels(asm["collectives.hip"]).items()
          if k.startswith("_ZN4snac11copy_kernelI") and "Lb0E" in k and shape in k}
    assert ks, shape
    for name, lines in ks.items():
        # the extra dwords of the units of one tile (4 per lane in these shapes)
        assert _longest_unwaited_run(lines, "global_load_dword") >= 4, f"{name}: misaligned loads serialised"


# reduce_kernel<N, T, CP, ALIGNED, SMALL, ROLL>
REDUCE_NAME = re.compile(r"_ZN4snac13reduce_kernelILi(\d+)ENS_\d+(\w+?)ELi(\d)ELb([01])ELb([01])ELb([01])EEEv")


def _reduce_kernels(asm: str) -> dict[tuple, list[str]]:
    out = {}
    for k, v in _kernels(asm).items():
        m = REDUCE_NAME.match(k)
        if m:
            n, t, cp, a, small, roll = m.groups()
            out[(int(n), t, int(cp), a == "1", small == "1", roll == "1")] = v
    return out


def test_reduce_kernel_set(asm):
    ks = _reduce_kernels(asm["collectives.hip"])
    # N = 1..16, two types: four cache policies aligned and two generic at
    # 16 KiB tiles, aligned and generic small tiles; the rolling form for
    # bf16 N=8 at 16 KiB tiles only
    assert len([k for k in ks if not k[5]]) == 16 * 2 * 8
    assert sorted(k for k in ks if k[5]) == sorted(
        [(8, "BF16", cp, True, False, True) for cp in range(4)] + [(8, "BF16", cp, False, False, True) for cp in (0, 1)])


def test_rolling_allreduce_tile_keeps_four_loads_in_flight(asm):
    # the bf16 AllReduce of 8 ranks, aligned, every cache policy: the tile's
    # 32 loads per lane go out at most 4 without a wait, and each wait leaves
    # 2-3 in flight (the two-buffer form waits 8 times, leaving 4-7)
    ks = {k: v for k, v in _reduce_kernels(asm["collectives.hip"]).items() if k[5] and k[3]}
    assert len(ks) == 4
    for key, lines in ks.items():
        code = [l.strip() for l in lines if l.strip() and not l.strip().startswith(";")]
        loads = [i for i, l in enumerate(code) if l.startswith("buffer_load_dwordx4")]
        assert len(loads) == 32, f"{key}: {len(loads)} tile loads"
        region = code[loads[0]:loads[-1] + 1]
        waits = [int(m.group(1)) for m in (re.search(r"vmcnt\((\d+)\)", l) for l in region
                                           if l.startswith("s_waitcnt")) if m]
        assert len(waits) >= 24 and set(waits) <= {2, 3}, f"{key}: waits {waits}"
        assert _longest_unwaited_run(region, "buffer_load_dwordx4") <= 4, f"{key}: loads hoisted"


def test_misaligned_reduce_tile_issues_every_load_first(asm):
    # generic reduce kernels: the 16 KiB-tile form keeps a source's 4 units
    # per lane in flight, the small-tile form every source's unit
    ks = {k: v for k, v in _reduce_kernels(asm["collectives.hip"]).items() if not k[3]}
    assert len(ks) == 98
    for (n, t, cp, a, small, roll), lines in ks.items():
        want = n if small else 4
        assert _longest_unwaited_run(lines, "global_load_dword") >= want, \
            f"reduce N={n} {t} cp={cp} small={small} roll={roll}: misaligned loads serialised"


def test_misaligned_256_thread_copy_uses_dpp_shifts(asm):
    ks = {k: v for k, v in _kernels(asm["collectives.hip"]).items()
          if k.startswith("_ZN4snac11copy_kernelI") and "Lb0ELi256ELj16384E" in k}
    assert ks
    for name, lines in ks.items():
        assert any("wave_shl:1" in l for l in lines), f"{name}: no DPP lane shift"


def test_tile_counter_fetch_stays_in_flight(asm):
    ks = {k: v for k, v in _kernels(asm["collectives.hip"]).items()
          if (REDUCE_NAME.match(k) and REDUCE_NAME.match(k).group(5) == "0")
          or (k.startswith("_ZN4snac11copy_kernelI") and "Lj16384E" in k)}
    assert len(ks) >= 6 + 16 * 2 * 6
    probes = {k: v for k, v in _kernels(asm["probes.hip"]).items() if "probe_kernel" in k}
    assert len(probes) == 12
    ks.update(probes)
    for name, lines in ks.items():
        text = "\n".join(lines)
        assert "flat_atomic" not in text and "scratch_" not in text, name
        code = [l.strip() for l in lines if l.strip() and not l.strip().startswith(";")]
        fetch = [i for i, l in enumerate(code) if l.startswith("global_atomic_add_x2") and " sc0" in l]
        assert fetch, f"{name}: no counter fetch"
        i = fetch[0]
        assert not any(l.startswith("v_mbcnt") for l in code[max(0, i - 8):i]), f"{name}: fetch folded wave-wide"
        assert not any(re.match(r"s_waitcnt\s+vmcnt\(0\)", l) for l in code[i + 1:i + 4]), \
            f"{name}: waits for the tile fetch at once"
