"""Determinism of every kernel: the same inputs give the same bits over ten
calls, and again when each workgroup is launched with extra dynamic LDS that
lowers the number resident per CU (FA_TEST_EXTRA_LDS, read once per process,
so those runs happen in a child process).  No kernel accumulates through
atomics or in an order that depends on scheduling, so occupancy must not
change a single bit; the outputs are NaN-poisoned before each call, so an
element left unwritten would show as well.
"""
import json
import os
import subprocess
import sys
import tempfile
import time

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# name: (kind, B, Hq, Hkv, Nq, Nk, d, causal).  The grids hold more
# workgroups than the 768 (prefill) or 512 (backward) slots of a fully
# occupied GPU, so lowering the occupancy changes which workgroups run
# together and in what order.
CASES = {
    "bf16_gqa_causal": ("fwd", 2, 16, 4, 4096, 4096, 128, True),
    "bf16_d64_ragged": ("fwd", 8, 8, 8, 1000, 1000, 64, False),
    "fp8": ("fwd8", 2, 16, 16, 4096, 4096, 128, False),
    "decode": ("fwd", 4, 32, 8, 1, 4000, 128, True),
    "bwd_causal_d128": ("bwd", 4, 8, 4, 4096, 4096, 128, True),
    "bwd_d64": ("bwd", 8, 8, 8, 1000, 1000, 64, False),
}
TIMED = "bf16_gqa_causal"


def _bits(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    return t.cpu().numpy()


def compute(name, seed=11):
    """One call of the case's entry point on seeded inputs; returns the
    output bit patterns by name."""
    import exact_attention_105_amd as fa
    from synth.inputs import make_grad_output, make_inputs
    kind, B, Hq, Hkv, Nq, Nk, d, causal = CASES[name]
    dev = torch.device("cuda:0")
    dtype = "e4m3" if kind == "fwd8" else "bf16"
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed)
    if dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(torch.float8_e4m3fn)
    q, k, v = conv(x["q"]), conv(x["k"]), conv(x["v"])
    scale = d ** -0.5
    out = torch.full((B, Hq, Nq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=dev)
    o, l = fa.fwd(q, k, v, causal=causal, scale=scale, descale=x.get("descale"), out=out, lse=lse)
    res = {"O": o, "LSE": l}
    if kind == "bwd":
        do = conv(make_grad_output(B, Hq, Nq, d, seed))
        grads = [torch.full(t.shape, float("nan"), dtype=torch.bfloat16, device=dev) for t in (q, k, v)]
        dq, dk, dv = fa.bwd(q, k, v, o, l, do, causal=causal, scale=scale, dq=grads[0], dk=grads[1], dv=grads[2])
        res.update(dQ=dq, dK=dk, dV=dv)
    torch.cuda.synchronize()
    return {key: _bits(t) for key, t in res.items()}


def time_case(name, reps=20):
    """Average seconds per forward call of a case (inputs reused)."""
    import exact_attention_105_amd as fa
    from synth.inputs import make_inputs
    kind, B, Hq, Hkv, Nq, Nk, d, causal = CASES[name]
    dev = torch.device("cuda:0")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", 5)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[t]).view(np.int16)).to(dev).view(torch.bfloat16)
               for t in ("q", "k", "v"))
    for _ in range(5):
        fa.fwd(q, k, v, causal=causal, scale=d ** -0.5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fa.fwd(q, k, v, causal=causal, scale=d ** -0.5)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


def _child(out_path):
    import exact_attention_105_amd as fa
    fa.load()
    res = {f"{name}/{key}": a for name in CASES for key, a in compute(name).items()}
    np.savez(out_path, **res)
    with open(out_path + ".json", "w") as f:
        json.dump({"time_s": time_case(TIMED), "extra": os.environ.get("FA_TEST_EXTRA_LDS")}, f)


if __name__ == "__main__" and len(sys.argv) == 3 and sys.argv[1] == "--child":
    _child(sys.argv[2])
    sys.exit(0)


pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    assert os.environ.get("FA_TEST_EXTRA_LDS") is None, "the in-process runs must use the default launch"
    import exact_attention_105_amd as fa
    fa.load()


@pytest.mark.parametrize("name", list(CASES))
def test_ten_calls_identical(name):
    print(f"determinism: ten calls of {name} {CASES[name]}", flush=True)
    first = compute(name)
    for i in range(9):
        again = compute(name)
        for key in first:
            assert np.array_equal(first[key], again[key]), f"{name}: {key} differs on call {i + 2}"


@pytest.mark.parametrize("extra", [40 << 10, 96 << 10])
def test_lower_occupancy_identical(extra):
    """Each workgroup launched with `extra` bytes of unused dynamic LDS: the
    d = 128 prefill kernels' 32 KiB become 72 KiB (two workgroups per CU
    instead of three) or 128 KiB (one), and the backward kernels' likewise
    (the hook caps static plus dynamic LDS at 128 KiB)."""
    print(f"determinism under lower occupancy: FA_TEST_EXTRA_LDS={extra}", flush=True)
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "child.npz")
        env = dict(os.environ, FA_TEST_EXTRA_LDS=str(extra))
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--child", path], env=env, cwd=ROOT,
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        child = dict(np.load(path))
        with open(path + ".json") as f:
            meta = json.load(f)
    for name in CASES:
        ref = compute(name)
        for key, a in ref.items():
            assert np.array_equal(a, child[f"{name}/{key}"]), f"{name}: {key} changes under FA_TEST_EXTRA_LDS={extra}"
    # the hook took effect: one resident workgroup per CU instead of three is slower
    base = time_case(TIMED)
    print(f"  {TIMED}: {base * 1e6:.1f} us per call by default, {meta['time_s'] * 1e6:.1f} us with "
          f"{extra} bytes of extra LDS", flush=True)
    if extra >= (96 << 10):
        assert meta["time_s"] > 1.15 * base, "extra dynamic LDS did not lower the occupancy"
