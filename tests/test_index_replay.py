"""Host replay of the kernels' index arithmetic (tests/index_replay.cpp).

The workgroup orders and copy clamps live in csrc/fa_index.hpp as functions
compiled for both host and device; this builds a host program around those
same functions and runs it over whole grids of the five workloads and of 200
random shapes: every order must be a bijection onto its work units, and every
K/V (or Q/dO) row a copy fetches must lie inside its tensor.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_105_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "index_replay.cpp")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_index_replay(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "index_replay")
    # host-only compile: the program calls no GPU function
    subprocess.run([cc, "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O2", "-std=c++17",
                    "-I", CSRC, SRC, "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe, "200"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert " 0 failures" in r.stdout
