"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small problems and the GPT-2-shaped and decode workloads are compared element
by element over the whole output.  The longer full-size workloads are compared
over complete heads (every row of the first and last head, and of the last
head of the first key/value group under grouped-query attention) and on
sampled rows of other heads, plus properties that hold at any size.  Tolerances are in
gpu_util.py.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_105_amd import FaError, fwd
from gpu_util import (compare_bf16, complete_heads, head_rows, oracle_ref, run_gpu, sample_rows, say,
                      to_device)
from synth.inputs import CONFIGS, generate, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_105_amd as fa
    fa.load()


# (B, Hq, Hkv, Nq, Nk, d, causal): several tiles, ragged tails, GQA/MQA,
# Nq != Nk in both directions (bottom-right causal), single key, decode rows.
SMALL = [
    (1, 2, 2, 128, 128, 64, False),
    (2, 3, 3, 300, 300, 64, True),
    (2, 3, 3, 300, 300, 128, False),
    (1, 4, 2, 257, 257, 128, True),
    (2, 4, 1, 200, 333, 64, True),
    (1, 2, 2, 333, 200, 128, True),
    (1, 2, 2, 333, 200, 64, False),
    (1, 2, 2, 129, 1, 64, False),
    (1, 2, 2, 129, 1, 128, True),
    (3, 8, 2, 1, 1000, 128, True),
    (2, 8, 8, 1, 77, 64, False),
    (1, 1, 1, 1, 1, 64, False),
    (1, 2, 2, 64, 64, 128, True),
    (1, 2, 2, 65, 65, 64, True),
    (2, 2, 2, 190, 70, 64, False),
    (1, 3, 1, 512, 512, 128, True),
]


@pytest.mark.parametrize("shape", SMALL, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}Nq{s[3]}Nk{s[4]}d{s[5]}{'c' if s[6] else 'n'}"
                                               for s in SMALL])
def test_small_bf16(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    say(f"case {shape}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", 1000 + sum(shape))
    scale = 1.0 / math.sqrt(d)
    o, lse = run_gpu(x, "bf16", causal, scale)
    o_ref, lse_ref = oracle_ref(x, "bf16", causal, scale)
    compare_bf16(o, lse, o_ref, lse_ref, str(shape))


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.0, 1e-3])
def test_scale_values(scale):
    x = make_inputs(1, 2, 2, 150, 150, 64, "bf16", 31)
    for causal in (False, True):
        o, lse = run_gpu(x, "bf16", causal, scale)
        o_ref, lse_ref = oracle_ref(x, "bf16", causal, scale)
        compare_bf16(o, lse, o_ref, lse_ref, f"scale={scale} causal={causal}")


def test_hand_cases_padded():
    """The hand-worked 2x2 / 3x3 cases, zero-padded to d = 64 (padding leaves scores unchanged)."""
    from oracle_pins import _scalar, load_hand_cases
    from synth.inputs import f32_to_bf16_bits
    for case in load_hand_cases():
        n = len(case["q"])
        pad = lambda vals: np.pad(np.array([_scalar(t) for t in vals], dtype=np.float32).reshape(1, 1, n, 1),
                                  ((0, 0), (0, 0), (0, 0), (0, 63)))
        x = {"q": f32_to_bf16_bits(pad(case["q"])), "k": f32_to_bf16_bits(pad(case["k"])),
             "v": f32_to_bf16_bits(pad(case["v"]))}
        for causal in (False, True):
            o, lse = run_gpu(x, "bf16", causal, 1.0)
            o_ref, lse_ref = oracle_ref(x, "bf16", causal, 1.0)
            compare_bf16(o, lse, o_ref, lse_ref, f"{case['name']} causal={causal}")
            key = "causal" if causal else "non_causal"
            want = np.array([_scalar(t) for t in case[key]["o"]])
            # bf16 inputs (ln 2, ln 3 rounded) and bf16 output keep O near the closed form
            assert np.abs(o[0, 0, :, 0] - want).max() < 0.1
            assert np.all(o[0, 0, :, 1:] == 0.0)


def test_no_keys_and_no_queries():
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 5, 64, device=dev).bfloat16()
    k = torch.empty(1, 2, 0, 64, device=dev, dtype=torch.bfloat16)
    out = torch.full((1, 2, 5, 64), 7.0, device=dev, dtype=torch.bfloat16)
    lse = torch.full((1, 2, 5), 7.0, device=dev)
    # rows to compute and no key: an argument error, outputs untouched
    with pytest.raises(FaError) as e:
        fwd(q, k, k.clone(), causal=False, out=out, lse=lse)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
    q0 = torch.empty(1, 2, 0, 64, device=dev, dtype=torch.bfloat16)
    kk = torch.randn(1, 2, 7, 64, device=dev).bfloat16()
    o, lse = fwd(q0, kk, kk.clone(), causal=True)
    assert o.shape == (1, 2, 0, 64)


def test_errors_leave_outputs_untouched():
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 8, 96, device=dev).bfloat16()
    out = torch.full((1, 2, 8, 96), 7.0, device=dev, dtype=torch.bfloat16)
    lse = torch.full((1, 2, 8), 7.0, device=dev)
    with pytest.raises(FaError) as e:
        fwd(q, q.clone(), q.clone(), out=out, lse=lse)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_deterministic():
    x = make_inputs(2, 4, 2, 700, 700, 128, "bf16", 77)
    a = run_gpu(x, "bf16", True, 0.088)
    b = run_gpu(x, "bf16", True, 0.088)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_lse_optional():
    x = make_inputs(1, 2, 2, 100, 100, 64, "bf16", 78)
    q, k, v = to_device(x, "bf16")
    o1, l1 = fwd(q, k, v, causal=True)
    o2, l2 = fwd(q, k, v, causal=True, return_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)


# Keys whose norms grow along the sequence: each row's running maximum keeps
# rising, so the kernels' lazily moved exponent reference has to move many
# times after the first key tile (N(0,1) inputs almost never need that).
GROWING = [
    (1, 2, 2, 700, 700, 128, False),
    (1, 2, 2, 700, 700, 128, True),
    (2, 2, 1, 513, 600, 64, False),
    (1, 3, 3, 600, 600, 64, True),
]


def _growing_keys(x, growth):
    from synth.inputs import f32_to_bf16_bits
    k = (x["k"].astype(np.uint32) << 16).view(np.float32)
    nk = k.shape[2]
    ramp = (1.0 + growth * np.arange(nk, dtype=np.float32) / nk)[None, None, :, None]
    x = dict(x)
    x["k"] = f32_to_bf16_bits(k * ramp).reshape(k.shape)
    return x


@pytest.mark.parametrize("shape", GROWING, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}Nq{s[3]}Nk{s[4]}d{s[5]}{'c' if s[6] else 'n'}"
                                                 for s in GROWING])
def test_reference_moves_mid_row(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    say(f"case {shape}")
    x = _growing_keys(make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", 2000 + sum(shape)), growth=9.0)
    scale = 1.0 / math.sqrt(d)
    # the inputs do what they are for: in the last query row, the maximum
    # score (log2 units) of the last 32 keys exceeds that of the first 32 by
    # more than 12, so its reference moves after the first tile
    q = (x["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = (x["k"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s2 = q[0, 0, -1] @ k[0, 0].T * scale / math.log(2)
    assert s2[-32:].max() - s2[:32].max() > 12, (s2[:32].max(), s2[-32:].max())
    o, lse = run_gpu(x, "bf16", causal, scale)
    o_ref, lse_ref = oracle_ref(x, "bf16", causal, scale)
    compare_bf16(o, lse, o_ref, lse_ref, str(shape))


# ------------------------------------------------------------------ full-size workloads
BF16_CONFIGS = ["tiny", "gpt2", "gpt2_causal", "long16k_causal", "gqa_causal", "gqa_decode"]
# compared with the oracle over the whole output (the oracle finishes them in
# seconds); the longer workloads are compared over complete heads -- every
# query tile and the whole causal staircase of those heads -- plus sampled
# rows of the other heads
WHOLE_OUTPUT = ("tiny", "gpt2", "gpt2_causal", "gqa_decode")


@pytest.mark.parametrize("name", BF16_CONFIGS)
def test_config_bf16(name):
    cfg = CONFIGS[name]
    say(f"config {name}: {cfg}")
    x = generate(cfg)
    o, lse = run_gpu(x, "bf16", cfg.causal, cfg.scale)
    assert np.all(np.isfinite(o)), "unwritten or non-finite outputs"
    assert np.all(np.isfinite(lse))
    if name in WHOLE_OUTPUT:
        o_ref, lse_ref = oracle_ref(x, "bf16", cfg.causal, cfg.scale)
        compare_bf16(o, lse, o_ref, lse_ref, f"{name} (whole output)")
    else:
        heads = complete_heads(cfg.B, cfg.Hq, cfg.Hkv)
        rows = head_rows(cfg.Hq, cfg.Nq, heads)
        o_ref, lse_ref = oracle_ref(x, "bf16", cfg.causal, cfg.scale, rows=rows)
        compare_bf16(o.reshape(-1, cfg.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref,
                     f"{name} (complete heads {heads}, {rows.size} rows)")
        others = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq) if (b, h) not in heads]
        pick = np.random.default_rng(cfg.seed).choice(len(others), size=min(6, len(others)), replace=False)
        rows = sample_rows(cfg.B, cfg.Hq, cfg.Nq, seed=cfg.seed, heads=[others[i] for i in sorted(pick)])
        o_ref, lse_ref = oracle_ref(x, "bf16", cfg.causal, cfg.scale, rows=rows)
        compare_bf16(o.reshape(-1, cfg.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref,
                     f"{name} ({rows.size} sampled rows of other heads)")
    if cfg.causal and cfg.Nq == cfg.Nk:
        # row 0 sees only key 0: O_0 = V_0 exactly, for every head
        from oracle_pins import bf16_to_f64_torch
        v0 = bf16_to_f64_torch(x["v"][:, :, 0, :]).numpy()            # [B, Hkv, d]
        g = cfg.Hq // cfg.Hkv
        assert np.array_equal(o[:, :, 0, :], np.repeat(v0, g, axis=1))


# ------------------------------------------------------------------ FP8 (E4M3)
FP8_SMALL = [
    (1, 2, 2, 128, 128, False),
    (2, 3, 3, 300, 300, True),
    (1, 4, 2, 257, 190, True),
    (1, 2, 2, 190, 257, False),
    (2, 8, 2, 1, 700, True),
    (1, 2, 2, 100, 1, False),
]


@pytest.mark.parametrize("shape", FP8_SMALL, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}Nq{s[3]}Nk{s[4]}{'c' if s[5] else 'n'}"
                                                  for s in FP8_SMALL])
def test_small_fp8(shape):
    from gpu_util import compare_fp8, fp8_lse_bound
    B, Hq, Hkv, Nq, Nk, causal = shape
    say(f"fp8 case {shape}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, 128, "e4m3", 2000 + sum(shape))
    scale = 1.0 / math.sqrt(128)
    o, lse = run_gpu(x, "e4m3", causal, scale)
    o_ref, lse_ref = oracle_ref(x, "e4m3", causal, scale)
    compare_fp8(o, lse, o_ref, lse_ref, f"fp8 {shape}", lse_bound=fp8_lse_bound(x, None, scale))
    # rows without any visible key follow the convention exactly
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))


def test_fp8_negative_scale():
    from gpu_util import compare_fp8, fp8_lse_bound
    x = make_inputs(1, 2, 2, 150, 150, 128, "e4m3", 2100)
    o, lse = run_gpu(x, "e4m3", True, -0.05)
    o_ref, lse_ref = oracle_ref(x, "e4m3", True, -0.05)
    compare_fp8(o, lse, o_ref, lse_ref, "fp8 scale=-0.05", lse_bound=fp8_lse_bound(x, None, -0.05))


def test_config_fp8():
    from gpu_util import compare_fp8, fp8_lse_bound
    cfg = CONFIGS["fp8"]
    say(f"config fp8: {cfg}")
    x = generate(cfg)
    o, lse = run_gpu(x, "e4m3", cfg.causal, cfg.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    heads = complete_heads(cfg.B, cfg.Hq, cfg.Hkv)
    rows = head_rows(cfg.Hq, cfg.Nq, heads)
    o_ref, lse_ref = oracle_ref(x, "e4m3", cfg.causal, cfg.scale, rows=rows)
    compare_fp8(o.reshape(-1, cfg.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref,
                f"fp8 (complete heads {heads}, {rows.size} rows)", lse_bound=fp8_lse_bound(x, rows, cfg.scale))
    others = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq) if (b, h) not in heads]
    pick = np.random.default_rng(cfg.seed).choice(len(others), size=min(6, len(others)), replace=False)
    rows = sample_rows(cfg.B, cfg.Hq, cfg.Nq, seed=cfg.seed, heads=[others[i] for i in sorted(pick)])
    o_ref, lse_ref = oracle_ref(x, "e4m3", cfg.causal, cfg.scale, rows=rows)
    compare_fp8(o.reshape(-1, cfg.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref,
                f"fp8 ({rows.size} sampled rows of other heads)", lse_bound=fp8_lse_bound(x, rows, cfg.scale))


# ------------------------------------------------------------------ few query rows (decode path)
# bf16, d = 128, Nq <= 16 runs the grouped-query packed decode kernel:
# packed rows Nq*G up to and beyond one 32-row tile, key counts that are not
# multiples of the 32-key tile or smaller than the four per-wave key ranges.
DECODE = [
    (2, 32, 8, 1, 8192, True),
    (3, 8, 2, 1, 1000, False),
    (2, 4, 4, 1, 1, True),
    (1, 4, 1, 1, 31, False),
    (1, 8, 1, 2, 33, True),
    (2, 16, 2, 5, 100, True),
    (1, 16, 4, 16, 300, True),
    (1, 16, 4, 16, 300, False),
    (1, 8, 8, 3, 129, True),
    (1, 2, 2, 16, 16, True),
    (1, 2, 1, 7, 4, True),
]


@pytest.mark.parametrize("shape", DECODE, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}Nq{s[3]}Nk{s[4]}{'c' if s[5] else 'n'}"
                                               for s in DECODE])
def test_decode_bf16(shape):
    B, Hq, Hkv, Nq, Nk, causal = shape
    say(f"decode case {shape}")
    x = make_inputs(B, Hq, Hkv, Nq, Nk, 128, "bf16", 3000 + sum(shape))
    scale = 1.0 / math.sqrt(128)
    o, lse = run_gpu(x, "bf16", causal, scale)
    o_ref, lse_ref = oracle_ref(x, "bf16", causal, scale)
    compare_bf16(o, lse, o_ref, lse_ref, f"decode {shape}")
