"""Pins of the exact-attention oracle against facts fixed outside the oracle.

Each ``pin_*`` function takes an oracle handle (``oracle.OracleLib``) and
raises AssertionError when the oracle disagrees with something the pages or
the mathematics fix: closed-form hand cases, invariants of softmax attention,
brute force in plain Python, a library softmax on the CPU, and the codecs'
specifications.  ``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on copies of the oracle with
planted mistakes and requires every mistake to be caught.

The definition pinned is page "FlashAttention (DE)" (systems-analysis.info),
section "Problematik der Standard-Attention"; the tiled recurrence is the
same page's section "Online-Softmax-Berechnung".
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from synth.inputs import f32_to_bf16_bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def bf16_to_f64_torch(bits: np.ndarray) -> torch.Tensor:
    """Decode bfloat16 bit patterns with torch (a library routine, not the oracle's)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def e4m3_to_f64_torch(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double()


def torch_attention(q, k, v, causal, scale):
    """softmax(scale Q K^T + mask) V and logsumexp with torch on the CPU in float64.

    q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] float64 tensors.  Fully masked rows give
    O = 0 and LSE = -inf (the oracle's convention for a row with no key).
    """
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(q, k.transpose(-1, -2).contiguous())
    if causal:
        i = torch.arange(Nq).view(-1, 1)
        j = torch.arange(Nk).view(1, -1)
        s = s.masked_fill(j > i + (Nk - Nq), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)
    return torch.matmul(p, v), lse


def rand_bf16(B, Hq, Hkv, Nq, Nk, d, seed):
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed)
    return x["q"], x["k"], x["v"]


def _scalar(x):
    if isinstance(x, (int, float)):
        return float(x)
    x = x.strip()
    if x.startswith("ln "):
        return math.log(float(x[3:]))
    if "/" in x:
        a, b = x.split("/")
        return float(a) / float(b)
    return float(x)


def load_hand_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        return json.load(f)["cases"]


def close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_ninf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        diff = np.where(both_ninf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), f"{what}: non-finite mismatch"
    worst = float(diff.max()) if diff.size else 0.0
    assert worst <= tol, f"{what}: max abs diff {worst:.3e} > {tol:.1e}"


# -------------------------------------------------------------------- pins
def pin_hand_cases(orc):
    """Closed-form 2x2 and 3x3 cases (golden fixture, worked by hand)."""
    for case in load_hand_cases():
        n = len(case["q"])
        q = np.array([_scalar(x) for x in case["q"]]).reshape(1, 1, n, 1)
        k = np.array([_scalar(x) for x in case["k"]]).reshape(1, 1, n, 1)
        v = np.array([_scalar(x) for x in case["v"]]).reshape(1, 1, n, 1)
        for key, causal in (("non_causal", False), ("causal", True)):
            want_o = np.array([_scalar(x) for x in case[key]["o"]])
            want_l = np.array([_scalar(x) for x in case[key]["lse"]])
            for bk in (0, 1, 2):
                o, lse = orc.attention(q, k, v, causal=causal, scale=1.0, dtype="f64", block_keys=bk)
                close(o.reshape(-1), want_o, 1e-12, f"{case['name']} {key} O (block {bk})")
                close(lse.reshape(-1), want_l, 1e-12, f"{case['name']} {key} LSE (block {bk})")


def pin_probs_rows(orc):
    """Each materialised P row is a probability vector; masked keys get exactly 0."""
    q, k, v = rand_bf16(1, 2, 2, 13, 17, 16, 7001)
    for causal in (False, True):
        for row in (0, 5, 12, 13 + 12):
            p = orc.probs_row(q, k, v, causal=causal, scale=0.25, row=row)
            assert np.all(p >= 0.0)
            assert abs(p.sum() - 1.0) < 1e-13, f"row {row} sums to {p.sum()}"
            if causal:
                i = row % 13
                assert np.all(p[i + (17 - 13) + 1:] == 0.0), "masked keys must have P = 0"
                assert np.all(p[: i + (17 - 13) + 1] > 0.0)


def pin_library_softmax(orc):
    """Tiny inputs: the oracle equals torch.softmax(S) @ V in float64 on the CPU."""
    for causal in (False, True):
        for (Nq, Nk) in ((9, 11), (11, 9), (16, 16)):
            q, k, v = rand_bf16(2, 4, 2, Nq, Nk, 8, 7002 + Nq)
            scale = 1.0 / math.sqrt(8)
            o, lse = orc.attention(q, k, v, causal=causal, scale=scale)
            to, tl = torch_attention(bf16_to_f64_torch(q), bf16_to_f64_torch(k),
                                     bf16_to_f64_torch(v), causal, scale)
            close(o, to.numpy(), 1e-12, f"O vs torch causal={causal} {Nq}x{Nk}")
            close(lse, tl.numpy(), 1e-12, f"LSE vs torch causal={causal} {Nq}x{Nk}")


def pin_bruteforce_python(orc):
    """Plain-Python loops with math.exp on a tiny float64 problem (GQA 2:1)."""
    rng = np.random.default_rng(7003)
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 4, 5, 3
    q = rng.standard_normal((B, Hq, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    scale = 0.7
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, causal=causal, scale=scale, dtype="f64")
        for h in range(Hq):
            for i in range(Nq):
                vis = [j for j in range(Nk) if (not causal) or j <= i + Nk - Nq]
                s = {j: scale * sum(q[0, h, i, t] * k[0, 0, j, t] for t in range(d)) for j in vis}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in vis}
                tot = sum(w.values())
                for t in range(d):
                    want = sum(w[j] * v[0, 0, j, t] for j in vis) / tot
                    assert abs(o[0, h, i, t] - want) < 1e-12
                assert abs(lse[0, h, i] - (mx + math.log(tot))) < 1e-12


def pin_constant_v(orc):
    """V = c everywhere gives O = c for every visible row."""
    q, k, _ = rand_bf16(2, 2, 2, 20, 20, 16, 7004)
    v = np.full(k.shape, 0x3FE0, dtype=np.uint16)          # 1.75 exactly
    for causal in (False, True):
        o, _ = orc.attention(q, k, v, causal=causal, scale=0.25)
        close(o, np.full(o.shape, 1.75), 1e-13, "constant V")


def pin_single_key(orc):
    """Nk = 1: O = V_0 and LSE = scale * <q, k_0>."""
    q, k, v = rand_bf16(1, 3, 3, 6, 1, 16, 7005)
    o, lse = orc.attention(q, k, v, causal=False, scale=0.3)
    tq, tk, tv = bf16_to_f64_torch(q), bf16_to_f64_torch(k), bf16_to_f64_torch(v)
    close(o, tv.expand(1, 3, 6, 16).numpy(), 1e-14, "Nk=1 O")
    want = 0.3 * (tq * tk).sum(-1)
    close(lse, want.numpy(), 1e-12, "Nk=1 LSE")


def pin_causal_first_row(orc):
    """Causal, Nq = Nk: row 0 sees only key 0, so O_0 = V_0 and LSE_0 = s_00."""
    q, k, v = rand_bf16(2, 2, 2, 10, 10, 16, 7006)
    o, lse = orc.attention(q, k, v, causal=True, scale=0.25)
    tq, tk, tv = bf16_to_f64_torch(q), bf16_to_f64_torch(k), bf16_to_f64_torch(v)
    close(o[:, :, 0, :], tv[:, :, 0, :].numpy(), 1e-14, "causal row 0")
    close(lse[:, :, 0], (0.25 * (tq[:, :, 0] * tk[:, :, 0]).sum(-1)).numpy(), 1e-12, "row 0 LSE")


def pin_zero_query(orc):
    """Q = 0: P is uniform over the visible keys -- prefix means and LSE = ln(count)."""
    _, k, v = rand_bf16(1, 2, 2, 12, 15, 8, 7007)
    for Nq in (15, 12):
        q = np.zeros((1, 2, Nq, 8), dtype=np.uint16)
        tv = bf16_to_f64_torch(v).numpy()
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, causal=causal, scale=0.5)
            for i in range(Nq):
                cnt = (i + 15 - Nq + 1) if causal else 15
                close(o[0, :, i], tv[0, :, :cnt].mean(axis=1), 1e-13, f"Q=0 row {i}")
                close(lse[0, :, i], np.full(2, math.log(cnt)), 1e-13, f"Q=0 LSE row {i}")


def pin_key_permutation(orc):
    """Non-causal attention is invariant to permuting keys and values together."""
    q, k, v = rand_bf16(1, 2, 2, 7, 19, 16, 7008)
    perm = np.random.default_rng(1).permutation(19)
    o1, l1 = orc.attention(q, k, v, causal=False, scale=0.25)
    o2, l2 = orc.attention(q, k[:, :, perm], v[:, :, perm], causal=False, scale=0.25)
    close(o1, o2, 1e-13, "key permutation O")
    close(l1, l2, 1e-13, "key permutation LSE")
    # ... and is not invariant to permuting the values alone
    o3, _ = orc.attention(q, k, v[:, :, perm], causal=False, scale=0.25)
    assert np.abs(o3 - o1).max() > 1e-3


def pin_linear_in_v(orc):
    """O is linear in V."""
    rng = np.random.default_rng(7009)
    q = rng.standard_normal((1, 2, 8, 4))
    k = rng.standard_normal((1, 2, 11, 4))
    v1 = rng.standard_normal((1, 2, 11, 4))
    v2 = rng.standard_normal((1, 2, 11, 4))
    for causal in (False, True):
        oa, _ = orc.attention(q, k, v1, causal=causal, scale=0.5, dtype="f64")
        ob, _ = orc.attention(q, k, v2, causal=causal, scale=0.5, dtype="f64")
        oc, _ = orc.attention(q, k, v1 - 2.0 * v2, causal=causal, scale=0.5, dtype="f64")
        close(oc, oa - 2.0 * ob, 1e-12, "linearity in V")


def pin_lse_bounds(orc):
    """max_j s_ij <= LSE_i <= max_j s_ij + ln(#visible keys)."""
    q, k, v = rand_bf16(1, 2, 2, 16, 16, 16, 7010)
    tq, tk = bf16_to_f64_torch(q), bf16_to_f64_torch(k)
    s = 0.25 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    for causal in (False, True):
        _, lse = orc.attention(q, k, v, causal=causal, scale=0.25)
        for i in range(16):
            cnt = i + 1 if causal else 16
            mx = s[0, :, i, :cnt].max(dim=-1).values.numpy()
            assert np.all(lse[0, :, i] >= mx - 1e-12)
            assert np.all(lse[0, :, i] <= mx + math.log(cnt) + 1e-12)
            if cnt > 1:
                assert np.all(lse[0, :, i] > mx + 1e-9)


def pin_gqa_repeat(orc):
    """GQA with g query heads per KV head equals MHA with K/V repeated g times."""
    q, k, v = rand_bf16(2, 6, 2, 9, 12, 16, 7011)
    for causal in (False, True):
        o1, l1 = orc.attention(q, k, v, causal=causal, scale=0.25)
        o2, l2 = orc.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1),
                               causal=causal, scale=0.25)
        close(o1, o2, 0.0, "GQA vs repeated MHA O")
        close(l1, l2, 0.0, "GQA vs repeated MHA LSE")


def pin_gqa_grouping(orc):
    """Query heads 0..g-1 read KV head 0, heads g..2g-1 read KV head 1 (consecutive groups)."""
    q, k, v = rand_bf16(1, 4, 2, 5, 6, 8, 7012)
    v = v.copy()
    v[:, 0] = 0x3F80      # 1.0
    v[:, 1] = 0x4040      # 3.0
    o, _ = orc.attention(q, k, v, causal=False, scale=0.25)
    close(o[:, :2], np.full(o[:, :2].shape, 1.0), 1e-14, "heads 0,1 -> kv 0")
    close(o[:, 2:], np.full(o[:, 2:].shape, 3.0), 1e-14, "heads 2,3 -> kv 1")


def pin_decode_is_last_causal_row(orc):
    """Nq = 1 causal (bottom-right aligned) equals the last row of the square causal problem."""
    q, k, v = rand_bf16(2, 4, 2, 24, 24, 16, 7013)
    of, lf = orc.attention(q, k, v, causal=True, scale=0.25)
    od, ld = orc.attention(q[:, :, -1:], k, v, causal=True, scale=0.25)
    close(od[:, :, 0], of[:, :, -1], 0.0, "decode O")
    close(ld[:, :, 0], lf[:, :, -1], 0.0, "decode LSE")
    on, ln_ = orc.attention(q[:, :, -1:], k, v, causal=False, scale=0.25)
    close(on, od, 0.0, "decode causal == non-causal")


def pin_fully_masked_rows(orc):
    """Causal with Nq > Nk: the first Nq - Nk rows see no key (O = 0, LSE = -inf)."""
    q, k, v = rand_bf16(1, 2, 2, 10, 4, 8, 7014)
    o, lse = orc.attention(q, k, v, causal=True, scale=0.25)
    assert np.all(o[:, :, :6] == 0.0)
    assert np.all(np.isneginf(lse[:, :, :6]))
    to, tl = torch_attention(bf16_to_f64_torch(q), bf16_to_f64_torch(k), bf16_to_f64_torch(v),
                             True, 0.25)
    close(o[:, :, 6:], to[:, :, 6:].numpy(), 1e-12, "visible rows O")
    close(lse[:, :, 6:], tl[:, :, 6:].numpy(), 1e-12, "visible rows LSE")


def pin_tiled_equals_naive(orc):
    """The online-softmax recurrence reproduces the naive definition for any block size."""
    cases = [(1, 2, 2, 37, 37, True), (1, 2, 1, 37, 37, False), (2, 2, 2, 21, 45, True),
             (1, 2, 2, 30, 11, True), (1, 1, 1, 1, 130, False)]
    for (B, Hq, Hkv, Nq, Nk, causal) in cases:
        q, k, v = rand_bf16(B, Hq, Hkv, Nq, Nk, 16, 7015 + Nq + Nk)
        on, ln_ = orc.attention(q, k, v, causal=causal, scale=0.25)
        for bc in (1, 7, 64, Nk):
            ot, lt = orc.attention(q, k, v, causal=causal, scale=0.25, block_keys=bc)
            close(ot, on, 1e-12, f"tiled O bc={bc} {Nq}x{Nk} causal={causal}")
            close(lt, ln_, 1e-12, f"tiled LSE bc={bc} {Nq}x{Nk} causal={causal}")


def pin_scale_applied(orc):
    """The scale multiplies the scores: scale c with Q equals scale 1 with c*Q."""
    rng = np.random.default_rng(7016)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 2, 9, 4))
    v = rng.standard_normal((1, 2, 9, 4))
    o1, l1 = orc.attention(q, k, v, causal=True, scale=1.7, dtype="f64")
    o2, l2 = orc.attention(1.7 * q, k, v, causal=True, scale=1.0, dtype="f64")
    close(o1, o2, 1e-12, "scale O")
    close(l1, l2, 1e-12, "scale LSE")


def pin_e4m3_inputs(orc):
    """E4M3 codes with per-tensor scales equal float64 inputs decoded by torch and scaled."""
    x = make_inputs(1, 2, 2, 10, 14, 16, "e4m3", 7017)
    ds = x["descale"]
    assert all(s != 1.0 for s in ds)
    o, lse = orc.attention(x["q"], x["k"], x["v"], causal=True, scale=0.25, dtype="e4m3",
                           descale=ds)
    qf = (e4m3_to_f64_torch(x["q"]) * ds[0]).numpy()
    kf = (e4m3_to_f64_torch(x["k"]) * ds[1]).numpy()
    vf = (e4m3_to_f64_torch(x["v"]) * ds[2]).numpy()
    o2, l2 = orc.attention(qf, kf, vf, causal=True, scale=0.25, dtype="f64")
    close(o, o2, 1e-13, "e4m3 O")
    close(lse, l2, 1e-13, "e4m3 LSE")


def pin_rows_subset(orc):
    """Selecting rows returns exactly those rows of the full result."""
    q, k, v = rand_bf16(2, 4, 2, 11, 13, 16, 7018)
    of, lf = orc.attention(q, k, v, causal=True, scale=0.25)
    rows = np.array([0, 5, 43, 87, 12, 60])
    o, lse = orc.attention(q, k, v, causal=True, scale=0.25, rows=rows)
    close(o, of.reshape(-1, 16)[rows], 0.0, "row subset O")
    close(lse, lf.reshape(-1)[rows], 0.0, "row subset LSE")


def pin_bf16_decoder(orc):
    """All 65536 bfloat16 codes decode as (-1)^s 2^(e-127) (1 + m/128) (subnormal: 2^-126 m/128)."""
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(codes, "bf16")
    s = (codes >> 15) & 1
    e = (codes >> 7) & 0xFF
    m = (codes & 0x7F).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 128.0, -126),
                   np.ldexp(1.0 + m / 128.0, e.astype(np.int64) - 127))
    want = np.where(s == 1, -mag, mag)
    fin = e != 0xFF
    assert np.array_equal(got[fin], want[fin])
    inf = (e == 0xFF) & (m == 0)
    assert np.array_equal(got[inf], np.where(s[inf] == 1, -np.inf, np.inf))
    assert np.all(np.isnan(got[(e == 0xFF) & (m != 0)]))


def pin_e4m3_decoder(orc):
    """All 256 E4M3 codes decode per the OCP definition (bias 7, max 448, S.1111.111 = NaN)."""
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = orc.decode(codes, "e4m3", 1.0)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert math.isnan(got[c])
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert got[c] == (-mag if s else mag), f"code {c:#04x}"
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    scaled = orc.decode(codes[:0x7F], "e4m3", 0.5)
    assert np.array_equal(scaled, got[:0x7F] * 0.5)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
