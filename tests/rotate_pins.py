"""Pins of the incoherent-processing oracle (rotate_oracle.c) against things
other than itself: scipy's Hadamard matrix and numpy's matrix product, the
orthogonality that makes the rotation harmless to Q K^T (page
"FlashAttention-3 (DE)", systems-analysis.ru, technical innovation 3),
brute force over every E4M3 code, torch's float8_e4m3fn conversion and the
input generator's independent encoder.

Each pin takes an oracle library (the default one, or a planted mutant) and
raises AssertionError when it disagrees."""
import math

import numpy as np
import scipy.linalg
import torch

from synth.inputs import f32_to_bf16_bits, f64_to_e4m3_codes


def signs_for(d, seed):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1.0, 1.0)


def dense_m(d, signs):
    """M = D H / sqrt(d) from scipy's Sylvester Hadamard matrix."""
    return (np.diag(signs) @ scipy.linalg.hadamard(d).astype(np.float64)) / math.sqrt(d)


def rpin_hadamard_entries_match_scipy_and_are_orthogonal(orc):
    for d in [1, 2, 4, 8, 16, 32, 64, 128]:
        h = np.array([[orc.hadamard_entry(i, j) for j in range(d)] for i in range(d)])
        assert np.array_equal(h, scipy.linalg.hadamard(d).astype(np.float64)), d
        assert np.array_equal(h @ h.T, d * np.eye(d)), d


def rpin_order_two_by_hand(orc):
    h = [[orc.hadamard_entry(i, j) for j in range(2)] for i in range(2)]
    assert h == [[1.0, 1.0], [1.0, -1.0]]


def rpin_rotation_equals_dense_product(orc):
    for d in [64, 128]:
        rng = np.random.default_rng(d)
        x = rng.standard_normal((37, d))
        s = signs_for(d, 7)
        y = orc.rotate(x, signs=s)
        assert np.allclose(y, x @ dense_m(d, s), rtol=0, atol=1e-12), d


def rpin_basis_vectors_give_signed_hadamard_rows(orc):
    for d in [64, 128]:
        s = signs_for(d, 8)
        y = orc.rotate(np.eye(d), signs=s)
        want = s[:, None] * scipy.linalg.hadamard(d) / math.sqrt(d)
        assert np.allclose(y, want, rtol=0, atol=1e-15), d


def rpin_rotation_preserves_inner_products_and_norms(orc):
    d = 128
    rng = np.random.default_rng(3)
    q = rng.standard_normal((50, d))
    k = rng.standard_normal((60, d))
    s = signs_for(d, 9)
    qr, kr = orc.rotate(q, signs=s), orc.rotate(k, signs=s)
    assert np.allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-11)        # Q K^T unchanged
    assert np.allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q, axis=1), rtol=1e-14)


def rpin_outlier_channel_is_spread_evenly(orc):
    """A single large feature becomes d values of equal magnitude."""
    d = 128
    x = np.zeros((1, d))
    x[0, 17] = 20.0
    y = orc.rotate(x, signs=signs_for(d, 1))
    assert np.allclose(np.abs(y), 20.0 / math.sqrt(d), rtol=0, atol=1e-14)


def rpin_no_rotation_is_identity_and_no_signs_is_plain_hadamard(orc):
    d = 64
    x = np.random.default_rng(4).standard_normal((5, d))
    assert np.array_equal(orc.rotate(x, rotate=False), x)
    assert np.allclose(orc.rotate(x), x @ scipy.linalg.hadamard(d) / 8.0, rtol=0, atol=1e-13)


def rpin_input_dtypes_decode_exactly(orc):
    d = 64
    xf = np.random.default_rng(5).standard_normal((6, d)).astype(np.float32)
    s = signs_for(d, 2)
    assert np.array_equal(orc.rotate(xf, signs=s), orc.rotate(xf.astype(np.float64), signs=s))
    bits = f32_to_bf16_bits(xf)
    widened = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(orc.rotate(bits, signs=s), orc.rotate(widened, signs=s))


def rpin_rejects_non_power_of_two(orc):
    try:
        orc.rotate(np.zeros((2, 96)))
    except ValueError:
        return
    raise AssertionError("a non-power-of-two width was accepted")


# ---------------------------------------------------------------- E4M3 encoder
FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def _values(orc):
    return {c: float(orc.decode(np.array([c], dtype=np.uint8), "e4m3")[0]) for c in FINITE}


def rpin_encoder_round_trips_every_finite_code(orc):
    values = _values(orc)
    for c in FINITE:
        got = orc.e4m3_encode(values[c])
        assert got == c or (values[c] == 0.0 and got in (0, 128) and (got >> 7) == (c >> 7)), c


def rpin_encoder_is_nearest_with_ties_to_even_brute_force(orc):
    values = _values(orc)

    def brute_force(v):
        return min(FINITE, key=lambda c: (abs(values[c] - v), (c & 1), c))   # nearest, then even code

    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(3000) * 50, rng.standard_normal(1000) * 0.01,
                           rng.uniform(-448, 448, 1000)])
    # exact midpoints between neighbouring positive codes, both signs
    mags = sorted(values[c] for c in range(127))
    mids = [(a + b) / 2 for a, b in zip(mags, mags[1:])]
    vals = np.concatenate([vals, mids, -np.array(mids)])
    for v in vals:
        if v == 0.0:
            continue
        c = orc.e4m3_encode(v)
        b = brute_force(v)
        assert values[c] == values[b] and (c & 0x80) == (0x80 if v < 0 else 0), (v, c, b)


def rpin_encoder_saturates(orc):
    assert orc.e4m3_encode(448.0) == 0x7E
    assert orc.e4m3_encode(1e6) == 0x7E
    assert orc.e4m3_encode(-1e6) == 0xFE
    assert orc.e4m3_encode(460.0) == 0x7E


def rpin_encoder_matches_torch_and_the_input_generator(orc):
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.05])
    ours = np.array([orc.e4m3_encode(x) for x in v], dtype=np.uint8)
    torch_codes = torch.from_numpy(v.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, torch_codes)
    assert np.array_equal(ours, f64_to_e4m3_codes(v))


def rpin_quantize_scale_and_extremes(orc):
    rng = np.random.default_rng(13)
    y = rng.standard_normal((40, 64)) * 3
    codes, s = orc.quantize_e4m3(y)
    amax = np.abs(y).max()
    assert s == amax / 448.0
    i = np.unravel_index(np.abs(y).argmax(), y.shape)
    assert codes[i] in (0x7E, 0xFE)
    dec = orc.decode(codes, "e4m3", s)
    # every value within half an E4M3 step of its decoded code (relative 2^-4 for normals)
    assert np.all(np.abs(dec - y) <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * s) + 1e-12)
    # the quantiser's codes are the encoder's codes of y / s
    assert np.array_equal(codes.reshape(-1), np.array([orc.e4m3_encode(v / s) for v in y.reshape(-1)], dtype=np.uint8))
    # the encoding step alone, with the same scale, gives the same codes
    assert np.array_equal(orc.encode_scaled(y, s), codes)
    # the largest magnitude negative: the scale comes from |min|
    yn = y.copy()
    yn[0, 0] = -10 * amax
    cn, sn = orc.quantize_e4m3(yn)
    assert sn == 10 * amax / 448.0 and cn[0, 0] == 0xFE
    z, s0 = orc.quantize_e4m3(np.zeros((3, 8)))
    assert s0 == 1.0 and np.all(z == 0)


RPINS = [v for k, v in sorted(globals().items()) if k.startswith("rpin_")]
