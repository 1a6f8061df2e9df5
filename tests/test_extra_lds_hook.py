"""The occupancy test hook (FA_TEST_EXTRA_LDS, used by
tests/test_determinism_gpu.py) on the CPU: for every static LDS size the
kernels declare, static plus the requested dynamic LDS never exceeds 128 KiB,
and a kernel already held to one workgroup per CU (the 128 KiB decode kernel)
gets none.  The hook reads the variable once per process, so each request
runs in a child process; no GPU call is made.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_attention_105_amd", "libfa.so")

# static LDS of the hooked kernels (bytes): d=64 prefill and dQ, d=128 prefill
# (bf16 and fp8), d=64 dK/dV, d=128 dK/dV by wave pairs, d=128 pipelined dQ,
# decode
STATIC = [16384, 32768, 34816, 41472, 49152, 131072]

CHILD = r"""
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
f = lib._ZN2fa14test_extra_ldsEm
f.restype = ctypes.c_size_t
f.argtypes = [ctypes.c_size_t]
print(" ".join(str(f(int(s))) for s in sys.argv[2:]))
"""


def extra_for(want):
    env = dict(os.environ)
    env.pop("FA_TEST_EXTRA_LDS", None)
    if want is not None:
        env["FA_TEST_EXTRA_LDS"] = str(want)
    r = subprocess.run([sys.executable, "-c", CHILD, LIB, *map(str, STATIC)], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return [int(x) for x in r.stdout.split()]


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.parametrize("want", [None, 0, 4096, 40 << 10, 96 << 10, 1 << 30, -5])
def test_extra_lds_stays_within_cap(want):
    got = extra_for(want)
    for s, e in zip(STATIC, got):
        if want is None or want <= 0:
            assert e == 0
        elif 2 * s > (160 << 10):
            assert e == 0, f"static {s}: one workgroup per CU already, got {e}"
        else:
            assert s + e <= (128 << 10), f"static {s} + extra {e} above 128 KiB"
            assert e == min(want, (128 << 10) - s)
