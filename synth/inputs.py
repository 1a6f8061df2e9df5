"""Seeded synthetic inputs for the attention forward pass.

This module is the only code that both the HIP path's callers and the oracle
consume.  It draws random numbers and encodes them into the byte formats the
kernels read; it holds none of the attention arithmetic.

Recipe (the same bytes go to the GPU and to the oracle):

* standard normals from ``numpy.random.Generator(PCG64(seed))`` in float32,
  drawn for Q, then K, then V, each in C order [B, H, N, d];
* bfloat16: round-to-nearest-even of each float32 value, kept as uint16 bit
  patterns (the upper half of the binary32 word);
* FP8 (OCP E4M3): a seeded 1 % of the H*d feature channels (pairs of head
  and feature index, the same set for Q, K and V, drawn with seed + 100) is
  multiplied by 20 to create outlier channels; each tensor then gets one
  float32 scale s = amax / 448 and codes sat(RNE(x / s)).  The kernels receive
  the codes and s; the oracle decodes the codes and multiplies by s.

Workload shapes follow the pages' examples: batch 16 x 12 heads x 2048 tokens
x head dim 64 (page "Flash Attention", 21medien.de, "Performance-Benchmarks";
the same page's SDPA example uses 12 heads of 2048 tokens with head dim 64),
16K-token long context (same section), grouped-query sharing (same page, key
techniques; page "FlashAttention 4", centron.de, compatibility section) and
FP8 with outlier channels (page "FlashAttention-3 (DE)", systems-analysis.ru,
section on low precision and incoherent processing).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

_CHUNK = 1 << 24


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str          # "bf16" or "e4m3"
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Attention FLOPs 4*B*Hq*Nq*Nk*d, halved for causal square problems."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        if self.causal and self.Nq == self.Nk:
            f /= 2.0
        return f

    @property
    def elt(self) -> int:
        return 2 if self.dtype == "bf16" else 1

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once; O (bf16) and LSE (fp32) written once."""
        q = self.B * self.Hq * self.Nq * self.d * self.elt
        kv = 2 * self.B * self.Hkv * self.Nk * self.d * self.elt
        o = self.B * self.Hq * self.Nq * self.d * 2
        lse = self.B * self.Hq * self.Nq * 4
        return q + kv + o + lse


CONFIGS = {
    c.name: c for c in [
        Config("tiny", 1, 2, 2, 128, 128, 64, False, "bf16", 105001),
        Config("gpt2", 16, 12, 12, 2048, 2048, 64, False, "bf16", 105002),
        Config("gpt2_causal", 16, 12, 12, 2048, 2048, 64, True, "bf16", 105002),
        Config("long16k_causal", 2, 16, 16, 16384, 16384, 128, True, "bf16", 105003),
        Config("gqa_causal", 4, 32, 8, 8192, 8192, 128, True, "bf16", 105004),
        Config("gqa_decode", 64, 32, 8, 1, 8192, 128, True, "bf16", 105014),
        # one sequence decoding against a 64K-token cache: 8 key/value heads,
        # far fewer than the GPU's 256 compute units unless the keys are split
        Config("gqa_decode_b1", 1, 32, 8, 1, 65536, 128, True, "bf16", 105015),
        Config("fp8", 4, 16, 16, 8192, 8192, 128, False, "e4m3", 105005),
    ]
}


def normals(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 standard normals in C order, drawn in fixed-size chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        b = flat[s:e].view(np.uint32).astype(np.uint64)
        nan = ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)
        r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
        r = np.where(nan, (b >> 16) | 0x40, r)
        out[s:e] = r.astype(np.uint16)
    return out.reshape(x.shape)


def f64_to_e4m3_codes(y: np.ndarray) -> np.ndarray:
    """Encode values as OCP E4M3 codes: round to nearest even, saturate at +-448.

    E4M3: bias 7, 3 mantissa bits, subnormal quantum 2^-9, normal quantum
    2^(e-3) for magnitudes in [2^e, 2^(e+1)), e >= -6; code S.1111.111 is NaN
    and is never produced.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    _, e = np.frexp(a)                      # a = f * 2^e with f in [0.5, 1)
    ex = np.maximum(e - 1, -6)              # floor(log2 a), clamped to the subnormal range
    quantum = np.ldexp(1.0, ex - 3)
    qv = np.minimum(np.rint(a / quantum) * quantum, 448.0)
    _, e2 = np.frexp(qv)
    ex2 = e2 - 1
    normal = qv >= 2.0 ** -6
    exp_field = np.where(normal, ex2 + 7, 0)
    mant = np.where(normal, np.rint((qv / np.ldexp(1.0, np.where(normal, ex2, 0)) - 1.0) * 8.0),
                    np.rint(qv / 2.0 ** -9))
    code = sign | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)
    return code.astype(np.uint8)


def quantise_e4m3(x: np.ndarray):
    """Per-tensor E4M3 quantisation: returns (codes uint8, scale float32 = amax/448)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    codes = np.empty(x.shape, dtype=np.uint8)
    flat, cflat = x.reshape(-1), codes.reshape(-1)
    for i in range(0, flat.size, _CHUNK):
        j = min(flat.size, i + _CHUNK)
        cflat[i:j] = f64_to_e4m3_codes(flat[i:j].astype(np.float64) / np.float64(s))
    return codes, s


def outlier_channels(seed: int, H: int, d: int, frac: float = 0.01) -> np.ndarray:
    """Flat indices h*d + t of the outlier feature channels (round(frac*H*d) of them)."""
    n = int(round(frac * H * d))
    rng = np.random.Generator(np.random.PCG64(seed + 100))
    return np.sort(rng.choice(H * d, size=n, replace=False))


def generate(cfg: Config, *, outlier_mult: float = 20.0):
    """Inputs for one configuration.

    Returns a dict with ``q``, ``k``, ``v`` (uint16 bfloat16 bits or uint8 E4M3
    codes, shapes [B,Hq,Nq,d] / [B,Hkv,Nk,d]) and ``descale`` (None for bf16,
    (sq, sk, sv) float32 for E4M3).
    """
    return make_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, cfg.dtype, cfg.seed,
                       outlier_mult=outlier_mult)


def make_float_inputs(B, Hq, Hkv, Nq, Nk, d, seed, *, outlier_mult: float = 20.0):
    """The float32 Q, K, V of the FP8 recipe before quantisation: normals with
    the outlier channels multiplied by ``outlier_mult``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qf = normals(rng, (B, Hq, Nq, d))
    kf = normals(rng, (B, Hkv, Nk, d))
    vf = normals(rng, (B, Hkv, Nk, d))
    # outlier channels are drawn over the key/value heads; a query head gets
    # the channels of the key/value head it reads (the same set when Hq == Hkv)
    ch = outlier_channels(seed, Hkv, d)
    hs, ts = ch // d, ch % d
    g = Hq // Hkv
    for t in (kf, vf):
        t[:, hs, :, ts] *= np.float32(outlier_mult)
    for gi in range(g):
        qf[:, hs * g + gi, :, ts] *= np.float32(outlier_mult)
    return qf, kf, vf


def make_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed, *, outlier_mult: float = 20.0):
    if dtype == "bf16":
        rng = np.random.Generator(np.random.PCG64(seed))
        qf = normals(rng, (B, Hq, Nq, d))
        kf = normals(rng, (B, Hkv, Nk, d))
        vf = normals(rng, (B, Hkv, Nk, d))
        return {"q": f32_to_bf16_bits(qf), "k": f32_to_bf16_bits(kf),
                "v": f32_to_bf16_bits(vf), "descale": None}
    if dtype != "e4m3":
        raise ValueError(f"unknown dtype {dtype}")
    qf, kf, vf = make_float_inputs(B, Hq, Hkv, Nq, Nk, d, seed, outlier_mult=outlier_mult)
    qc, sq = quantise_e4m3(qf)
    kc, sk = quantise_e4m3(kf)
    vc, sv = quantise_e4m3(vf)
    return {"q": qc, "k": kc, "v": vc, "descale": (float(sq), float(sk), float(sv))}


def make_grad_output(B, Hq, Nq, d, seed):
    """The upstream gradient dO of a backward-pass workload: float32 standard
    normals from PCG64(seed + 1000), rounded to bfloat16 (uint16 bits)."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    return f32_to_bf16_bits(normals(rng, (B, Hq, Nq, d)))


# Variable-length (packed) workloads: per-sequence query and key lengths.
VARLEN_WORKLOADS = {
    # 24 causal sequences, lengths log-uniform in [128, 8192] (seed 105020), 16 heads, d 128
    "varlen_mix": dict(n_seqs=24, lo=128, hi=8192, Hq=16, Hkv=16, d=128, causal=True, seed=105020),
    # one 8192-token sequence packed with 255 sequences of 128 tokens, causal, 16 heads, d 128
    "varlen_skew": dict(n_seqs=256, long=8192, short=128, Hq=16, Hkv=16, d=128, causal=True, seed=105021),
}


def workload_lengths(w):
    """Sequence lengths of a VARLEN_WORKLOADS entry: log-uniform (lo, hi) or
    one long sequence followed by n_seqs - 1 short ones."""
    if "long" in w:
        return np.array([w["long"]] + [w["short"]] * (w["n_seqs"] - 1), dtype=np.int64)
    return varlen_lengths(w["n_seqs"], w["lo"], w["hi"], w["seed"])


def varlen_lengths(n_seqs, lo, hi, seed):
    """Sequence lengths, log-uniform in [lo, hi], from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi + 1), size=n_seqs))).astype(np.int64).clip(lo, hi)


def make_varlen_inputs(lens_q, lens_k, Hq, Hkv, d, seed):
    """Packed bf16 inputs: q [sum lens_q, Hq, d], k and v [sum lens_k, Hkv, d]
    (float32 standard normals from PCG64(seed), in that order, rounded to
    bf16) and the int32 offsets cu_q, cu_k."""
    rng = np.random.Generator(np.random.PCG64(seed))
    tq, tk = int(np.sum(lens_q)), int(np.sum(lens_k))
    q = f32_to_bf16_bits(normals(rng, (tq, Hq, d)))
    k = f32_to_bf16_bits(normals(rng, (tk, Hkv, d)))
    v = f32_to_bf16_bits(normals(rng, (tk, Hkv, d)))
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return {"q": q, "k": k, "v": v, "cu_q": cu_q, "cu_k": cu_k}
