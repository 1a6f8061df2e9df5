"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The oracle sources are compiled once more with
-fsanitize=address,undefined (no recovery), and every pin of the attention,
backward and rotation oracles runs against that build in a child process
that preloads the ASan runtime.  A heap or stack overflow, a use after free,
a signed overflow, a misaligned or null access, or a shift out of range in
any oracle path the pins reach ends the child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

from oracle.oracle import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from oracle.oracle import OracleLib
from oracle_pins import PINS
from bwd_pins import BPINS
from rotate_pins import RPINS
orc = OracleLib({lib!r})
n = 0
for pin in list(PINS) + list(BPINS) + list(RPINS):
    pin(orc)
    n += 1
print("pins passed:", n)
"""


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True,
                             check=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.fail("gcc's libasan.so not found")
    lib = build(force=True, out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = libasan + ((":" + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    out = r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "pins passed:" in out, out[-4000:]


def test_the_sanitized_build_reports_a_planted_overflow(tmp_path):
    """The same set-up catches a planted one-past-the-end read in the oracle
    (oracle_decode reading n + 1 elements), so a clean run above means
    something."""
    from oracle.oracle import _SRC
    src = open(_SRC).read()
    old = "for (int64_t x = 0; x < n; ++x) dst[x] = load_elem(src, dtype, x, descale);"
    assert src.count(old) == 1
    mutant = tmp_path / "attn_oracle_overflow.c"
    mutant.write_text(src.replace(old, "for (int64_t x = 0; x <= n; ++x) dst[x] = load_elem(src, dtype, x, descale);"))
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True,
                             check=True).stdout.strip()
    lib = build(force=True, src=str(mutant), out=str(tmp_path / "liboracle_overflow.so"), sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = libasan + ((":" + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "import numpy as np\n"
            "from oracle.oracle import OracleLib\n"
            f"orc = OracleLib({lib!r})\n"
            "x = np.arange(8, dtype=np.uint16)\n"
            "orc.decode(x, 'bf16')\n")
    r = subprocess.run([sys.executable, "-c", code], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stdout, r.stdout[-2000:]
