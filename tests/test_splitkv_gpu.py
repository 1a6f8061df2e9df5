"""GPU parity of fa_fwd_splitkv (decode with the keys split over several
workgroups and merged) against the fp64 oracle, with the bf16 tolerances of
gpu_util.py; n_splits = 1 must equal fa_fwd bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_105_amd import FaError, default_splits, fwd, fwd_splitkv
from gpu_util import compare_bf16, say, to_device
from synth.inputs import CONFIGS, generate, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_105_amd as fa
    fa.load()


def run(x, causal, scale, n_splits):
    q, k, v = to_device(x, "bf16")
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, l = fwd_splitkv(q, k, v, causal=causal, scale=scale, n_splits=n_splits, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), l.cpu().double().numpy()


# (B, Hq, Hkv, Nq, Nk, causal, n_splits)
CASES = [
    (1, 32, 8, 1, 4096, True, 16),
    (1, 32, 8, 1, 4096, True, 7),        # splits that do not divide the tiles
    (2, 8, 8, 4, 3000, True, 5),         # Nq > 1: bottom-right causal per row
    (1, 16, 1, 16, 1000, False, 3),      # MQA, 256 packed rows (8 row tiles)
    (1, 8, 2, 1, 100, True, 64),         # more splits than key tiles: empty splits
    (1, 8, 2, 2, 1, False, 4),           # one key
    (1, 32, 8, 1, 65536, True, 256),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}N{c[3]}x{c[4]}{'c' if c[5] else ''}s{c[6]}" for c in CASES])
def test_splitkv_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, causal, ns = case
    x = make_inputs(B, Hq, Hkv, Nq, Nk, 128, "bf16", 900 + Nk + ns)
    scale = 1.0 / math.sqrt(128)
    say(f"splitkv {case}")
    o, lse = run(x, causal, scale, ns)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], causal=causal, scale=scale)
    compare_bf16(o, lse, o_ref, lse_ref, f"splitkv {case}")


def test_no_keys_is_an_argument_error():
    """Rows to compute and no key: FA_ERROR_INVALID_VALUE, outputs untouched."""
    dev = torch.device("cuda:0")
    q = torch.randn(1, 8, 3, 128, device=dev).bfloat16()
    k = torch.empty(1, 2, 0, 128, device=dev, dtype=torch.bfloat16)
    out = torch.full((1, 8, 3, 128), 7.0, device=dev, dtype=torch.bfloat16)
    lse = torch.full((1, 8, 3), 7.0, device=dev)
    with pytest.raises(FaError) as e:
        fwd_splitkv(q, k, k.clone(), causal=True, scale=0.1, n_splits=4, out=out, lse=lse)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_one_split_is_the_decode_kernel_bit_for_bit():
    x = make_inputs(2, 32, 8, 1, 5000, 128, "bf16", 31)
    o1, l1 = run(x, True, 0.088, 1)
    q, k, v = to_device(x, "bf16")
    o, l = fwd(q, k, v, causal=True, scale=0.088)
    torch.cuda.synchronize()
    assert np.array_equal(o1, o.float().cpu().double().numpy()) and np.array_equal(l1, l.cpu().double().numpy())


def test_small_batch_decode_workload_default_splits():
    """The B=1 64K-key decode workload with the default split count."""
    cfg = CONFIGS["gqa_decode_b1"]
    x = generate(cfg)
    ns = default_splits(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk)
    say(f"gqa_decode_b1 with {ns} splits")
    o, lse = run(x, cfg.causal, cfg.scale, None)
    o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], causal=cfg.causal, scale=cfg.scale)
    compare_bf16(o, lse, o_ref, lse_ref, "gqa_decode_b1")
