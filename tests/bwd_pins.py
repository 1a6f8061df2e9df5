"""Pins of the attention-backward oracle (``oracle/attn_bwd_oracle.c``).

Each ``bpin_*`` takes an oracle library (the real one or a mutant) and
raises AssertionError when the oracle disagrees with something fixed
independently of it:

* torch.autograd through a float64 softmax attention written with torch ops
  (a library differentiating the forward definition);
* central finite differences of L = sum(O * dO), with O from the forward
  oracle (the derivative by its definition);
* a pure-Python triple loop with math.exp on tiny inputs;
* invariants of the exact gradients: the dK rows of a key/value head sum to
  zero (each softmax Jacobian row sums to zero), the dV rows sum to the sum
  of dO over the rows that see a key, linearity in dO, a query that sees a
  single key has dQ = 0, scale 0 gives dQ = dK = 0 and dV = column means;
* grouped-query heads equal the same problem with K/V repeated per query
  head, the gradients of the copies summed;
* the row-subset dQ equals the same rows of the full result, and bf16 bit
  patterns give the same result as their float64 values.
"""
import math

import numpy as np
import torch

from synth.inputs import f32_to_bf16_bits


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _problem(B, Hq, Hkv, Nq, Nk, d, seed):
    q = _rand((B, Hq, Nq, d), seed)
    k = _rand((B, Hkv, Nk, d), seed + 1)
    v = _rand((B, Hkv, Nk, d), seed + 2)
    do = _rand((B, Hq, Nq, d), seed + 3)
    return q, k, v, do


def _torch_grads(q, k, v, do, causal, scale):
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    Kr, Vr = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
    S = scale * torch.matmul(Q, Kr.transpose(-1, -2).contiguous())
    Nq, Nk = q.shape[2], k.shape[2]
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        S = S.masked_fill(j > i + (Nk - Nq), float("-inf"))
    P = torch.softmax(S, dim=-1)
    P = torch.nan_to_num(P, nan=0.0)          # rows with no visible key
    O = torch.matmul(P, Vr)
    (O * torch.tensor(do)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def _close(a, b, tol, what):
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def bpin_matches_torch_autograd(orc):
    for (B, Hq, Hkv, Nq, Nk, d, causal, scale, seed) in [
        (1, 2, 1, 5, 7, 8, True, 0.3, 1),
        (2, 4, 2, 6, 6, 4, False, 0.5, 2),
        (1, 3, 3, 9, 4, 5, True, 0.7, 3),      # Nq > Nk: the first rows see no key
        (1, 2, 2, 1, 11, 8, True, 0.25, 4),    # a decode row
        (1, 2, 1, 4, 4, 6, False, -0.4, 5),    # negative scale
    ]:
        q, k, v, do = _problem(B, Hq, Hkv, Nq, Nk, d, seed)
        got = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype="f64")
        ref = _torch_grads(q, k, v, do, causal, scale)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            _close(a, b, 1e-12, f"{name} vs torch autograd {B, Hq, Hkv, Nq, Nk, d, causal}")


def bpin_central_finite_differences(orc):
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 4, 5, 3
    q, k, v, do = _problem(B, Hq, Hkv, Nq, Nk, d, 11)
    for causal in (False, True):
        scale = 0.6

        def loss(q_, k_, v_):
            o, _ = orc.attention(q_, k_, v_, causal=causal, scale=scale, dtype="f64")
            return float(np.sum(o * do))

        dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype="f64")
        h = 1e-5
        rng = np.random.default_rng(12)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(6):
                idx = tuple(int(rng.integers(0, n)) for n in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), \
                    f"d{name}{idx} causal={causal}: oracle {g[idx]!r} vs finite difference {fd!r}"


def bpin_brute_force_python(orc):
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 3, 4, 2
    q, k, v, do = _problem(B, Hq, Hkv, Nq, Nk, d, 21)
    scale, causal = 0.8, True
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        for i in range(Nq):
            vis = [j for j in range(Nk) if j <= i + (Nk - Nq)]
            if not vis:
                continue
            s = {j: scale * sum(q[0, h, i, t] * k[0, 0, j, t] for t in range(d)) for j in vis}
            m = max(s.values())
            z = sum(math.exp(s[j] - m) for j in vis)
            p = {j: math.exp(s[j] - m) / z for j in vis}
            dp = {j: sum(do[0, h, i, t] * v[0, 0, j, t] for t in range(d)) for j in vis}
            dsum = sum(p[j] * dp[j] for j in vis)
            for j in vis:
                ds = p[j] * (dp[j] - dsum)
                for t in range(d):
                    dq[0, h, i, t] += scale * ds * k[0, 0, j, t]
                    dk[0, 0, j, t] += scale * ds * q[0, h, i, t]
                    dv[0, 0, j, t] += p[j] * do[0, h, i, t]
    got = orc.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype="f64")
    for name, a, b in zip(("dQ", "dK", "dV"), got, (dq, dk, dv)):
        _close(a, b, 1e-13, f"{name} vs brute force")


def bpin_gradient_invariants(orc):
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 7, 9, 6
    q, k, v, do = _problem(B, Hq, Hkv, Nq, Nk, d, 31)
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=causal, scale=0.45, dtype="f64")
        # each softmax Jacobian row sums to zero, so the dK rows of a head do
        _close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-12, f"sum_j dK_j causal={causal}")
        # sum_j dV_j = sum over the group's rows that see a key of dO_i
        seen = np.array([(not causal) or (i + (Nk - Nq) >= 0) for i in range(Nq)])
        want = (do * seen[None, None, :, None]).reshape(B, Hkv, Hq // Hkv, Nq, d).sum(axis=(2, 3))
        _close(dv.sum(axis=2), want, 1e-12, f"sum_j dV_j causal={causal}")
        # linear in dO
        do2 = _rand(do.shape, 32)
        g1 = orc.attention_bwd(q, k, v, do, causal=causal, scale=0.45, dtype="f64")
        g2 = orc.attention_bwd(q, k, v, do2, causal=causal, scale=0.45, dtype="f64")
        g3 = orc.attention_bwd(q, k, v, 2.5 * do - do2, causal=causal, scale=0.45, dtype="f64")
        for a, b, c, name in zip(g1, g2, g3, ("dQ", "dK", "dV")):
            _close(c, 2.5 * a - b, 1e-12, f"{name} linear in dO causal={causal}")
    # causal with Nq == Nk: row 0 sees only key 0, so its dQ is exactly zero
    q, k, v, do = _problem(1, 2, 2, 5, 5, 4, 33)
    dq, _, _ = orc.attention_bwd(q, k, v, do, causal=True, scale=0.9, dtype="f64")
    _close(dq[:, :, 0], np.zeros((1, 2, 4)), 1e-15, "dQ of a row with one visible key")
    assert np.abs(dq[:, :, 1:]).max() > 1e-3, "dQ of rows with several keys must not vanish"


def bpin_scale_zero_and_empty(orc):
    q, k, v, do = _problem(1, 2, 1, 4, 6, 3, 41)
    dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=False, scale=0.0, dtype="f64")
    _close(dq, np.zeros_like(dq), 0.0, "dQ at scale 0")
    _close(dk, np.zeros_like(dk), 0.0, "dK at scale 0")
    # uniform P = 1/Nk: every key receives the mean of dO over all query rows of the group
    _close(dv, np.broadcast_to(do.sum(axis=(1, 2), keepdims=True) / 6, dv.shape), 1e-14, "dV at scale 0")
    # no keys at all
    q0, k0, v0, do0 = _problem(1, 2, 1, 3, 0, 4, 42)
    dq, dk, dv = orc.attention_bwd(q0, k0, v0, do0, causal=False, scale=0.5, dtype="f64")
    assert dq.shape == q0.shape and dk.shape == (1, 1, 0, 4) and not dq.any()
    # causal with Nq > Nk: the first Nq - Nk rows see nothing and get dQ = 0
    q1, k1, v1, do1 = _problem(1, 1, 1, 6, 3, 4, 43)
    dq, _, _ = orc.attention_bwd(q1, k1, v1, do1, causal=True, scale=0.5, dtype="f64")
    _close(dq[0, 0, :3], np.zeros((3, 4)), 0.0, "dQ of rows that see no key")
    assert np.abs(dq[0, 0, 4:]).max() > 1e-3


def bpin_gqa_equals_repeated_heads(orc):
    B, Hq, Hkv, Nq, Nk, d = 1, 6, 2, 5, 8, 4
    q, k, v, do = _problem(B, Hq, Hkv, Nq, Nk, d, 51)
    G = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=causal, scale=0.5, dtype="f64")
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        dq_r, dk_r, dv_r = orc.attention_bwd(q, kr, vr, do, causal=causal, scale=0.5, dtype="f64")
        _close(dq, dq_r, 1e-13, "dQ GQA vs repeated")
        _close(dk, dk_r.reshape(B, Hkv, G, Nk, d).sum(axis=2), 1e-13, "dK GQA vs repeated, summed")
        _close(dv, dv_r.reshape(B, Hkv, G, Nk, d).sum(axis=2), 1e-13, "dV GQA vs repeated, summed")


def bpin_row_subset_and_bf16_inputs(orc):
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 9, 13, 8
    q, k, v, do = _problem(B, Hq, Hkv, Nq, Nk, d, 61)
    bits = [f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v, do)]
    vals = [orc.decode(b, "bf16") for b in bits]
    for causal in (False, True):
        full_b = orc.attention_bwd(*bits, causal=causal, scale=0.35, dtype="bf16")
        full_f = orc.attention_bwd(*vals, causal=causal, scale=0.35, dtype="f64")
        for a, b, name in zip(full_b, full_f, ("dQ", "dK", "dV")):
            _close(a, b, 0.0, f"{name} from bf16 bits vs their float64 values")
        rows = [0, 5, 17, 35, 71, 8]
        sub = orc.bwd_dq_rows(*bits, causal=causal, scale=0.35, rows=rows, dtype="bf16")
        _close(sub, full_b[0].reshape(-1, d)[rows], 0.0, "dQ rows vs full dQ")


BPINS = [v for k, v in sorted(globals().items()) if k.startswith("bpin_")]
