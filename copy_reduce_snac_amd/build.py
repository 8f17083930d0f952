"""Build libsnac.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m copy_reduce_snac_amd.build          # build (always recompiles)

Each HIP source is compiled to an object in parallel, then linked into
``copy_reduce_snac_amd/libsnac.so``.  Flags:

* ``--offload-arch=gfx950``           MI355X only;
* ``-ffp-contract=off``               no fused multiply-add: every binary32 add
                                      and multiply rounds on its own;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``
                                      keep the compiler from forming packed
                                      fp32 instructions;
* no ``-ffast-math`` and no denormal flushing.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsnac.so")
SOURCES = ["api.hip", "collectives.hip", "pipeline.hip"]

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
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
