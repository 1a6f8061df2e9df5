"""The LDS copies (dma16 in fa_device.hpp) set M0 in inline asm and name it
as clobbered; M0 is a reserved register, so this is only safe while the
compiler keeps no value of its own in M0 across them.  This test compiles
every kernel source that uses dma16 to gfx950 assembly, with the library's
own flags, and checks that assumption on the code the compiler produced:

  * every mention of m0 is dma16's `s_mov_b32 m0, sN`, directly followed by
    its `global_load_lds_dwordx4` (so no compiler-placed M0 value exists);
  * every `global_load_lds_dwordx4` directly follows such a write;
  * no instruction that reads M0 implicitly appears (other LDS-DMA forms,
    GWS, append/consume, relative moves, interpolation, messages).

CPU only: hipcc cross-compiles, nothing runs on a GPU."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_105_amd import build

SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_fwd_decode.hip", "fa_bwd.hip"]
IMPLICIT_M0 = re.compile(r"^(ds_gws|ds_append|ds_consume|s_movrel|v_movrel|v_interp|s_sendmsg|ds_param_load|"
                         r"buffer_load_\w+\s.*\blds\b|global_load_lds_(?!dwordx4))")


def instructions(asm: str):
    """Instruction lines of the assembly (labels, directives, comments dropped)."""
    out = []
    for line in asm.split("\n"):
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        out.append(line)
    return out


def compile_to_asm(src: str, outdir: str) -> str:
    csrc = os.path.join(build.PKG, "csrc")
    out = os.path.join(outdir, src + ".s")
    cmd = [build.hipcc(), *build.HIPCC_FLAGS, *build.SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           "-I", build.INCLUDE, "-I", csrc, os.path.join(csrc, src), "-o", out]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm():
    if shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()):
        pytest.fail("hipcc not found")
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            texts = list(ex.map(lambda s: compile_to_asm(s, d), SOURCES))
    return dict(zip(SOURCES, texts))


@pytest.mark.parametrize("src", SOURCES)
def test_m0_is_only_set_for_the_lds_copies(asm, src):
    ins = instructions(asm[src])
    copies = 0
    for i, line in enumerate(ins):
        if re.search(r"\bm0\b", line):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", line), f"{src}: compiler use of m0: {line}"
            assert i + 1 < len(ins) and ins[i + 1].startswith("global_load_lds_dwordx4"), \
                f"{src}: m0 write not followed by the LDS copy: {line} / {ins[i + 1] if i + 1 < len(ins) else ''}"
        if line.startswith("global_load_lds_dwordx4"):
            copies += 1
            assert i > 0 and re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 1]), \
                f"{src}: LDS copy without its own m0 write: {ins[i - 1]} / {line}"
        assert not IMPLICIT_M0.match(line), f"{src}: instruction reading m0 implicitly: {line}"
    assert copies > 0, f"{src}: no LDS copies found"
