"""GPU parity of the backward pass (fa_bwd through the C ABI) against the
fp64 backward oracle.

The GPU runs its own forward pass for O and LSE, then the backward pass; the
oracle computes dQ, dK, dV from the same bfloat16 Q, K, V, dO by the chain
rule.  Small problems are compared element by element; the full-size
long-context workload on sampled dQ rows and on gradient invariants.

Tolerance, per gradient G in {dQ, dK, dV} with G_ref the oracle:
  rRMSE ||G - G_ref|| / ||G_ref|| <= 1e-2   and
  max |G - G_ref| <= 2e-2 * max |G_ref|.
The kernels round P and dS to bfloat16 before the matrix products (relative
error 2^-9 per element) and round the gradients to bfloat16 on output
(2^-9); D uses the bfloat16 O of the forward pass.  Independent roundings
of relative size 2^-9 give an rRMSE of a few 1e-3; the bounds leave a
factor of about 5 (rRMSE) and 10 (max) over that.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_105_amd import FaError, bwd, fwd
from gpu_util import say
from synth.inputs import CONFIGS, make_grad_output, make_inputs

pytestmark = pytest.mark.gpu

G_RRMSE = 1e-2
G_MAX_REL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_105_amd as fa
    fa.load()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def run(x, do_bits, causal, scale):
    q, k, v = (dev_bf16(x[n]) for n in ("q", "k", "v"))
    do = dev_bf16(do_bits)
    o, lse = fwd(q, k, v, causal=causal, scale=scale)
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    dk = torch.full(k.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    dv = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    bwd(q, k, v, o, lse, do, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().double().numpy() for t in (dq, dk, dv))


def compare(got, ref, what):
    # the largest gradient of the problem: the yardstick for a gradient whose
    # exact value is zero (a single visible key: dS = dP - D cancels exactly
    # in the oracle, up to fp32 summation order on the GPU)
    yard = max((float(np.abs(r).max()) for r in ref if r.size), default=0.0)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite values"
        if r.size == 0:
            continue
        scale = float(np.abs(r).max())
        if scale == 0.0:
            mx = float(np.abs(g).max()) / yard if yard > 0 else float(np.abs(g).max())
            say(f"  {what} {name}: exact zero, max|G| = {mx:.3e} of the largest gradient")
            assert mx <= G_MAX_REL * 1e-2, f"{what} {name}: {mx} of the largest gradient where the exact value is 0"
            continue
        rr = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        mx = float(np.abs(g - r).max()) / scale
        say(f"  {what} {name}: rRMSE={rr:.3e} max/|G|max={mx:.3e}")
        assert rr <= G_RRMSE, f"{what} {name}: rRMSE {rr} > {G_RRMSE}"
        assert mx <= G_MAX_REL, f"{what} {name}: max error {mx} of max|G| > {G_MAX_REL}"


# (B, Hq, Hkv, Nq, Nk, d, causal, scale or None): several tiles, ragged
# tails, GQA, Nq != Nk both ways, rows without keys, single key, one query.
CASES = [
    (1, 2, 2, 128, 128, 64, False, None),
    (1, 2, 1, 128, 128, 128, True, None),
    (1, 4, 2, 300, 300, 128, True, None),
    (2, 4, 4, 257, 190, 64, False, None),
    (1, 4, 1, 190, 257, 128, True, None),
    (1, 2, 2, 257, 130, 128, True, None),
    (1, 2, 2, 257, 130, 64, True, None),
    (1, 8, 2, 1, 300, 128, True, None),
    (1, 2, 1, 33, 1, 64, False, None),
    (1, 2, 2, 200, 200, 128, False, -0.09),
    (1, 2, 2, 100, 100, 64, True, 0.0),
    (2, 12, 12, 512, 512, 64, True, None),
    (1, 8, 2, 1024, 1024, 128, True, None),
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}N{c[3]}x{c[4]}d{c[5]}{'c' if c[6] else ''}{'' if c[7] is None else f's{c[7]}'}"
    for c in CASES])
def test_backward_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, d, causal, scale = case
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    seed = 7000 + B * 1000 + Nq + 3 * Nk + d
    x = make_inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed)
    do_bits = make_grad_output(B, Hq, Nq, d, seed)
    say(f"backward {case}")
    got = run(x, do_bits, causal, scale)
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], do_bits, causal=causal, scale=scale)
    compare(got, ref, str(case))


def test_backward_empty_sides():
    # no query rows: dK = dV = 0
    x = make_inputs(1, 2, 2, 0, 50, 128, "bf16", 99)
    do_bits = make_grad_output(1, 2, 0, 128, 99)
    say("backward Nq=0 Nk=50")
    dq, dk, dv = run(x, do_bits, True, 0.1)
    assert not dq.any() and not dk.any() and not dv.any()


def test_backward_no_keys_is_an_argument_error():
    """Query rows and no key: FA_ERROR_INVALID_VALUE (as for the forward),
    nothing launched, the gradients untouched."""
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 2, 40, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 2, 40), dtype=torch.float32, device=dev)
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    say("backward Nq=40 Nk=0")
    with pytest.raises(FaError) as e:
        bwd(q, k, k.clone(), o, lse, o.clone(), causal=True, scale=0.1, dq=dq)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.isnan(dq.float()).all()


def test_backward_full_size_long_context():
    """The 16K causal workload (B2 H16 N16384 d128): dQ on sampled rows against
    the oracle's row-local dQ; dK and dV through invariants of the exact
    gradients (the dK rows of a head sum to zero; the dV rows sum to the sum
    of dO over the head's query rows)."""
    cfg = CONFIGS["long16k_causal"]
    x = make_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, "bf16", cfg.seed)
    do_bits = make_grad_output(cfg.B, cfg.Hq, cfg.Nq, cfg.d, cfg.seed)
    say("backward full-size long-context")
    dq, dk, dv = run(x, do_bits, cfg.causal, cfg.scale)
    rows = np.random.default_rng(4).choice(cfg.B * cfg.Hq * cfg.Nq, size=512, replace=False)
    rows = np.concatenate([rows, [0, cfg.Nq - 1, cfg.Nq, cfg.B * cfg.Hq * cfg.Nq - 1]])
    ref = oracle.bwd_dq_rows(x["q"], x["k"], x["v"], do_bits, causal=cfg.causal, scale=cfg.scale, rows=rows)
    got = dq.reshape(-1, cfg.d)[rows]
    rr = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.abs(got - ref).max() / np.abs(ref).max())
    say(f"  sampled dQ rows: rRMSE={rr:.3e} max/|G|max={mx:.3e}")
    assert rr <= G_RRMSE and mx <= G_MAX_REL
    do = oracle.decode(do_bits, "bf16")
    G = cfg.Hq // cfg.Hkv
    sum_dk = dk.sum(axis=2)                                      # [B, Hkv, d]
    scale_dk = np.sqrt((dk ** 2).sum(axis=2))
    rel_k = float(np.abs(sum_dk).max() / scale_dk.max())
    want_dv = do.reshape(cfg.B, cfg.Hkv, G, cfg.Nq, cfg.d).sum(axis=(2, 3))
    rel_v = float(np.abs(dv.sum(axis=2) - want_dv).max() / np.abs(want_dv).max())
    say(f"  |sum_j dK_j| / ||dK col||: {rel_k:.3e}; |sum_j dV_j - sum_i dO_i| / max: {rel_v:.3e}")
    assert rel_k <= 2e-2, rel_k
    assert rel_v <= 1e-2, rel_v


BIG = [(32, 16, 16, 2048, 128, True), (16, 32, 8, 4300, 128, False), (64, 12, 12, 2048, 64, True)]


@pytest.mark.parametrize("shape", BIG, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else 'n'}" for s in BIG])
def test_backward_cache_sized_order(shape):
    """Problems whose streamed rows (Q and dO for dK/dV, K and V for dQ)
    exceed the 256 MiB memory-side cache run in a different workgroup order;
    one call per batch entry (small enough for the default order) must give
    the same bits, and sampled dQ rows must match the oracle."""
    B, Hq, Hkv, N, d, causal = shape
    assert B * Hq * N * d * 4 > (256 << 20) >= Hq * N * d * 4
    scale = 1.0 / math.sqrt(d)
    x = make_inputs(B, Hq, Hkv, N, N, d, "bf16", 9100 + N + d)
    do_bits = make_grad_output(B, Hq, N, d, 9100 + N + d)
    say(f"backward cache-sized order: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v = (dev_bf16(x[n]) for n in ("q", "k", "v"))
    do = dev_bf16(do_bits)
    o, lse = fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    for b in range(B):
        s = slice(b, b + 1)
        g1 = bwd(q[s], k[s], v[s], o[s], lse[s], do[s], causal=causal, scale=scale)
        for name, full, one in zip(("dQ", "dK", "dV"), (dq, dk, dv), g1):
            assert torch.equal(full[s], one), f"{name} of batch entry {b} differs"
    torch.cuda.synchronize()
    rows = np.random.default_rng(N + d).choice(B * Hq * N, size=256, replace=False)
    ref = oracle.bwd_dq_rows(x["q"], x["k"], x["v"], do_bits, causal=causal, scale=scale, rows=rows)
    got = dq.float().cpu().double().numpy().reshape(-1, d)[rows]
    rr = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.abs(got - ref).max() / np.abs(ref).max())
    say(f"  sampled dQ rows: rRMSE={rr:.3e} max/|G|max={mx:.3e}")
    assert rr <= G_RRMSE and mx <= G_MAX_REL
