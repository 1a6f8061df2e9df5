"""The input encoders (bfloat16 RNE, OCP E4M3 RNE with saturation) against torch (CPU only)."""
import numpy as np
import torch

from synth.inputs import (CONFIGS, f32_to_bf16_bits, f64_to_e4m3_codes, generate, make_inputs,
                          outlier_channels, quantise_e4m3)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, 1e-40, -1e-42], dtype=np.float32)]).astype(np.float32)
    # ties: values exactly halfway between two bfloat16 numbers
    base = np.arange(1, 2000, dtype=np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_e4m3_rne_matches_torch_in_range():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(100000) * 1e-2,
                        rng.standard_normal(1000) * 1e-4, [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10]])
    # exact midpoints between consecutive representable magnitudes
    mags = np.array(sorted({float(abs(v)) for v in torch.arange(0, 127, dtype=torch.uint8)
                            .view(torch.float8_e4m3fn).double().tolist()}))
    mids = (mags[:-1] + mags[1:]) / 2
    y = np.concatenate([y, mids, -mids]).astype(np.float64)
    got = f64_to_e4m3_codes(y)
    want = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # float32 conversion of y is exact for the midpoints and harmless elsewhere
    exact = y.astype(np.float32).astype(np.float64) == y
    assert np.array_equal(got[exact], want[exact])


def test_e4m3_saturates_and_never_nan():
    y = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e9, -1e9, -470.0])
    codes = f64_to_e4m3_codes(y)
    assert np.all((codes & 0x7F) == 0x7E)
    rng = np.random.default_rng(3)
    codes = f64_to_e4m3_codes(rng.standard_normal(100000) * 1000)
    assert not np.any((codes & 0x7F) == 0x7F)


def test_per_tensor_scale_uses_full_range():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 5, 7)).astype(np.float32)
    codes, s = quantise_e4m3(x)
    assert s == np.float32(np.abs(x).max() / np.float32(448.0))
    assert (codes & 0x7F).max() == 0x7E


def test_outlier_channels_recipe():
    ch = outlier_channels(105005, 16, 128)
    assert ch.size == 20 and np.unique(ch).size == 20
    x = make_inputs(1, 16, 16, 64, 64, 128, "e4m3", 105005)
    deq = torch.from_numpy(x["q"]).view(torch.float8_e4m3fn).double().numpy() * x["descale"][0]
    rms = np.sqrt((deq ** 2).mean(axis=(0, 2)))            # [H, d]
    flat = rms.reshape(-1)
    assert flat[ch].min() > 5 * np.median(flat)


def test_generation_is_deterministic():
    a = make_inputs(1, 2, 2, 33, 33, 64, "bf16", 9)
    b = make_inputs(1, 2, 2, 33, 33, 64, "bf16", 9)
    assert all(np.array_equal(a[n], b[n]) for n in ("q", "k", "v"))
    c = generate(CONFIGS["tiny"])
    assert c["q"].shape == (1, 2, 128, 64) and c["q"].dtype == np.uint16
