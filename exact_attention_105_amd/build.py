"""Build the HIP attention library (libfa.so) for gfx950 with hipcc.

Run as ``python -m exact_attention_105_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  The library is written next to this file so that it
travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_fwd_decode.hip", "fa_rotate.hip", "fa_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops (v_pk_*_f32) stay disabled
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions.  The prefill kernels schedule for instruction level
# parallelism (measured faster than the default occupancy-driven schedule, at
# the same three waves per SIMD).
SOURCE_FLAGS = {
    "fa_fwd_bf16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "fa_fwd_fp8.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False, jobs: int = 4, extra_flags=(), out: str = LIB,
          objdir: str | None = None, csrc: str = CSRC) -> str:
    """Compile every source for gfx950 and link the library (libfa.so by default).

    ``extra_flags`` are appended to every hipcc compile (e.g. -D tuning macros);
    ``out``/``objdir``/``csrc`` build a variant from another source tree into
    another place.  Returns the library path.
    """
    objdir = objdir or os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-I", INCLUDE, "-I", csrc, "-c",
               os.path.join(csrc, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


MICROBENCH = os.path.join(PKG, "microbench")
MICROBENCH_SOURCES = ["issue_rates.hip", "fp8_accumulation.hip", "coexec.hip", "phases.hip", "read_bw.hip"]


def build_microbench(verbose: bool = False) -> list:
    """Compile the stand-alone microbenchmark programs (microbench/*.hip)
    into microbench/bin/; returns their paths."""
    cc = hipcc()
    outdir = os.path.join(MICROBENCH, "bin")
    os.makedirs(outdir, exist_ok=True)
    procs, outs = [], []
    for src in MICROBENCH_SOURCES:
        out = os.path.join(outdir, src.replace(".hip", ""))
        outs.append(out)
        cmd = [cc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", os.path.join(MICROBENCH, src), "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    _drain(procs)
    return outs


def _drain(procs):
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            failed.append(f"--- {src}\n{out}")
        elif out and out.strip():
            sys.stderr.write(out)
    procs.clear()
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_microbench(verbose=True))
