"""Seeded sweep of random valid problem shapes through fa_fwd (bf16 and
fp8), fa_fwd_splitkv and the backward pass, each compared with the fp64
oracle under the tolerances of gpu_util.py.  The shapes mix batch sizes,
grouped-query ratios, ragged query and key lengths (Nq below, equal to and
above Nk), both head dims and both mask settings; they are drawn once from a
fixed seed, so every run checks the same cases.  The backward cases use the
gradient tolerances of test_bwd_gpu.py."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_105_amd import fwd_splitkv
from gpu_util import compare_bf16, compare_fp8, fp8_lse_bound, oracle_ref, run_gpu, say, to_device
from synth.inputs import make_grad_output, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_105_amd as fa
    fa.load()


def _draw(n, seed, nmax=420):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 2, 4]))
        Nq = int(rng.integers(1, nmax))
        Nk = int(rng.integers(1, nmax)) if rng.random() < 0.7 else Nq
        out.append((int(rng.integers(1, 3)), Hkv * g, Hkv, Nq, Nk, int(rng.choice([64, 128])),
                    bool(rng.random() < 0.5), float(rng.choice([1.0, -1.0, 0.5]))))
    return out


FWD = _draw(16, 105100)
FWD += _draw(12, 105110, 1400)       # longer rows: up to 11 query tiles and 44 key tiles


@pytest.mark.parametrize("case", FWD, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}s{c[7]}"
                                          for c in FWD])
def test_random_forward_bf16(case):
    B, Hq, Hkv, Nq, Nk, d, causal, smul = case
    say(f"case {case}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", 3000 + Nq + 7 * Nk)
    scale = smul / math.sqrt(d)
    o, lse = run_gpu(x, "bf16", causal, scale)
    o_ref, lse_ref = oracle_ref(x, "bf16", causal, scale)
    compare_bf16(o, lse, o_ref, lse_ref, str(case))


FP8 = [c for c in _draw(12, 105200) if c[5] == 128][:6]


@pytest.mark.parametrize("case", FP8, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}{'c' if c[6] else 'n'}" for c in FP8])
def test_random_forward_fp8(case):
    B, Hq, Hkv, Nq, Nk, d, causal, smul = case
    say(f"case {case}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "e4m3", 4000 + Nq + 7 * Nk)
    scale = smul / math.sqrt(d)
    o, lse = run_gpu(x, "e4m3", causal, scale)
    o_ref, lse_ref = oracle_ref(x, "e4m3", causal, scale)
    compare_fp8(o, lse, o_ref, lse_ref, str(case), lse_bound=fp8_lse_bound(x, None, scale))


def _draw_decode(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 4, 8]))
        out.append((int(rng.integers(1, 4)), Hkv * g, Hkv, int(rng.integers(1, 17)), int(rng.integers(1, 3000)),
                    bool(rng.random() < 0.5), int(rng.integers(1, 9))))
    return out


DEC = _draw_decode(8, 105300)


@pytest.mark.parametrize("case", DEC, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}{'c' if c[5] else 'n'}s{c[6]}"
                                          for c in DEC])
def test_random_splitkv(case):
    B, Hq, Hkv, Nq, Nk, causal, n_splits = case
    say(f"case {case}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, 128, "bf16", 5000 + Nq + 7 * Nk)
    scale = 1.0 / math.sqrt(128)
    q, k, v = to_device(x, "bf16")
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, l = fwd_splitkv(q, k, v, causal=causal, scale=scale, n_splits=n_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_ref(x, "bf16", causal, scale)
    compare_bf16(o.float().cpu().double().numpy(), l.cpu().double().numpy(), o_ref, lse_ref, str(case))


BWD = [c for c in _draw(10, 105400)][:6]
# six more at d = 128, the head dimension of the wave-pair dK/dV kernel (64-key
# blocks) and the software-pipelined dQ kernel
BWD += [c[:5] + (128,) + c[6:] for c in _draw(6, 105500)]
BWD += [c[:5] + (128,) + c[6:] for c in _draw(6, 105510, 700)]


@pytest.mark.parametrize("case", BWD, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{'c' if c[6] else 'n'}"
                                          for c in BWD])
def test_random_backward(case):
    from test_bwd_gpu import compare as bwd_compare, run as bwd_run
    B, Hq, Hkv, Nq, Nk, d, causal, smul = case
    say(f"case {case}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", 6000 + Nq + 7 * Nk)
    dob = make_grad_output(B, Hq, Nq, d, 6001 + Nq)
    scale = smul / math.sqrt(d)
    got = bwd_run(x, dob, causal, scale)
    refs = oracle.attention_bwd(x["q"], x["k"], x["v"], dob, causal=causal, scale=scale)
    bwd_compare(got, refs, str(case))
