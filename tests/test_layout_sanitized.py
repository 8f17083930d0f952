"""The layout engine's C++ header, compiled on the host with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and exercised on random
collectives (tests/cpp/test_layout.cpp).  CPU only."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
gxx = shutil.which("g++")


@pytest.mark.skipif(gxx is None, reason="g++ not available")
def test_layout_engine_under_sanitizers(tmp_path):
    exe = tmp_path / "test_layout"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "cpp", "test_layout.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:] + r.stdout[-1000:]
    assert "0 failures" in r.stdout
    leads = int(r.stdout.split(" jobs with a lead tile")[0].split()[-1])
    assert leads > 0, "no job got tiles cut to the destination grid: " + r.stdout
