"""Build libsnac.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m copy_reduce_snac_amd.build          # build (always recompiles)

Each HIP source is compiled to an object in parallel, then linked into
``copy_reduce_snac_amd/libsnac.so``; the device-API test fixture
(``tests/devapi/devapi_kernels.hip``) is linked into
``tests/devapi/libsnac_devtest.so``.  Flags:

* ``--offload-arch=gfx950``           MI355X only;
* ``-ffp-contract=off``               no fused multiply-add: every binary32 add
                                      and multiply rounds on its own;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``
                                      keep the compiler from forming packed
                                      fp32 instructions;
* no ``-ffast-math`` and no denormal flushing;
* ``collectives.hip`` and ``probes.hip`` also get
  ``-mllvm -amdgpu-atomic-optimizer-strategy=None`` (see SOURCE_FLAGS).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsnac.so")
SOURCES = ["api.hip", "collectives.hip", "pipeline.hip", "probes.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I" + INCLUDE,
]


# Test fixture: kernels that call the device-side API (include/snac_device.hpp)
# as a user's kernel would, with C launchers for the GPU tests.
DEVTEST_DIR = os.path.join(os.path.dirname(PKG), "tests", "devapi")
DEVTEST_SRC = os.path.join(DEVTEST_DIR, "devapi_kernels.hip")
DEVTEST_LIB = os.path.join(DEVTEST_DIR, "libsnac_devtest.so")


def _compile(jobs, verbose):
    """Run the hipcc commands of `jobs` [(name, cmd)] in parallel."""
    procs = []
    for name, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for name, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(name)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")


def _link(objs, out):
    tmp = out + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, out)


# Per-source flags.  collectives.hip and probes.hip: the compiler's atomic
# optimizer off.
# It turns an atomic on one address into a wave-wide reduction whose result
# it waits for at once; the shared tile counter's fetch must instead stay in
# flight while the current tile moves (TilePool in snac_device.hpp).
_NO_ATOMIC_OPT = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
SOURCE_FLAGS = {"collectives.hip": _NO_ATOMIC_OPT, "probes.hip": _NO_ATOMIC_OPT}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    jobs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append((src, [HIPCC, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]))
    dev_obj = os.path.join(BUILD, "devapi_kernels.o")
    jobs.append(("devapi_kernels.hip", [HIPCC, *DEVICE_FLAGS, "-c", DEVTEST_SRC, "-o", dev_obj]))
    _compile(jobs, verbose)
    _link(objs, LIB)
    _link([dev_obj], DEVTEST_LIB)
    if verbose:
        print(f"built {LIB} and {DEVTEST_LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
