"""The largest problems the entry points accept (every tensor just under 2^31
elements, 4 GiB of bf16), checked against closed forms, so that any 32-bit
overflow in a byte offset or row index would show.

Key side: one K/V head of 2^24 - 1 keys.  K is zero except one "spike" key
near the end (byte offset close to 4 GiB) whose score is 30, and V[k, :]
depends on bits 20-23 of k, so reading a row 2^23 keys (2 GiB) off would read
another value.  With every other score 0, O and LSE have closed forms:
  O = (e^30 V[s] + sum_{k != s, visible} V[k]) / (e^30 + n - 1),
  LSE = ln(e^30 + n - 1),  n the visible keys of the row.
Run through the decode kernel (Nq = 1, eight query heads packed), the
prefill kernel (Nq = 64, causal and not) and split-KV decode.

Query side: eight heads of 2^21 - 1 query rows each (Q and O 4 GiB), 64 keys.
K is zero except key 0, Q[h, r, :] = a/64 with a = ((h Nq + r) >> 18) mod 8,
scale 1, so key 0 scores 2a and every row has the closed form
  O = (e^{2a} V[0] + sum_{k >= 1} V[k]) / (e^{2a} + 63),  LSE = ln(e^{2a} + 63).
Every row of O and LSE is compared on the GPU (NaN-poisoned beforehand).

Backward: fa_bwd over the same 2^24 - 1 keys, its dV row of the spike against
its closed form and every gradient finite (outputs NaN-poisoned).
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_105_amd import fwd, fwd_splitkv
from gpu_util import BF16_MAX_ABS, LSE_MAX_ABS, say

pytestmark = pytest.mark.gpu

NK_MAX = (1 << 24) - 1          # 128 * NK_MAX = 2^31 - 128 elements
NQ_MAX = (1 << 21) - 1          # 8 heads * 128 * NQ_MAX = 2^31 - 1024 elements
SPIKE_SCORE = 30.0


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_105_amd as fa
    fa.load()


def v_of_key(k):
    """V[k, :] for key index k (exact in bf16): ((k >> 20) mod 16 - 7.5) / 16."""
    return (((k >> 20) & 15) - 7.5) / 16.0


def sum_v(n):
    """sum of v_of_key(k) over k < n, exactly."""
    full, part = divmod(n, 1 << 20)
    total = 0.0
    for blk in range(full):
        total += (1 << 20) * (((blk & 15) - 7.5) / 16.0)
    total += part * (((full & 15) - 7.5) / 16.0)
    return total


@pytest.fixture(scope="module")
def key_side():
    dev = torch.device("cuda:0")
    say(f"max-size key side: Nk = {NK_MAX}, K and V {NK_MAX * 128 * 2 / 2**30:.2f} GiB each")
    k = torch.zeros((1, 1, NK_MAX, 128), dtype=torch.bfloat16, device=dev)
    idx = torch.arange(NK_MAX, device=dev, dtype=torch.int64)
    vcol = ((((idx >> 20) & 15).to(torch.float32) - 7.5) / 16.0).to(torch.bfloat16)
    v = vcol.view(1, 1, NK_MAX, 1).expand(1, 1, NK_MAX, 128).contiguous()
    del idx, vcol
    torch.cuda.synchronize()
    return k, v


def expected_row(s, n_visible):
    """Closed-form O (one value for every column) and LSE of a row that sees
    keys 0 .. n_visible - 1, the spike s among them, with score 30 on s."""
    e = math.exp(SPIKE_SCORE)
    z = e + (n_visible - 1)
    o = (e * v_of_key(s) + (sum_v(n_visible) - v_of_key(s))) / z
    return o, math.log(z)


def check_rows(o, lse, exp_o, exp_lse, what):
    """o [rows, 128] bf16, lse [rows]; exp_o, exp_lse per row (float64 numpy)."""
    of = o.float().cpu().double().numpy()
    lf = lse.double().cpu().numpy()
    assert np.all(np.isfinite(of)) and np.all(np.isfinite(lf)), f"{what}: non-finite output"
    err = float(np.abs(of - np.asarray(exp_o)[:, None]).max())
    lerr = float(np.abs(lf - np.asarray(exp_lse)).max())
    say(f"  {what}: max|dO| = {err:.3e}, max|dLSE| = {lerr:.3e}")
    assert err <= BF16_MAX_ABS and lerr <= LSE_MAX_ABS, what


@pytest.mark.parametrize("path", ["decode", "splitkv", "prefill", "prefill_causal"])
def test_key_side_at_max(key_side, path):
    k, v = key_side
    dev = k.device
    s = NK_MAX - 100                        # visible to every row, also under the causal mask
    k[0, 0, s, :] = 1.0
    try:
        q_val = SPIKE_SCORE / 128.0         # 15/64: exact in bf16; score of the spike = 30
        if path in ("decode", "splitkv"):
            hq, nq = 8, 1
            kk, vv = k, v
        else:
            hq, nq = 1, 64
            kk, vv = k, v
        q = torch.full((1, hq, nq, 128), q_val, dtype=torch.bfloat16, device=dev)
        causal = path == "prefill_causal"
        out = torch.full((1, hq, nq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((1, hq, nq), float("nan"), dtype=torch.float32, device=dev)
        say(f"max-size key side, {path}: Hq={hq} Nq={nq} Nk={NK_MAX} causal={causal}")
        if path == "splitkv":
            o, l = fwd_splitkv(q, kk, vv, causal=False, scale=1.0, out=out, lse=lse)
        else:
            o, l = fwd(q, kk, vv, causal=causal, scale=1.0, out=out, lse=lse)
        torch.cuda.synchronize()
        exp_o, exp_l = [], []
        for h in range(hq):
            for i in range(nq):
                n_vis = NK_MAX - nq + i + 1 if causal else NK_MAX
                eo, el = expected_row(s, n_vis)
                exp_o.append(eo)
                exp_l.append(el)
        check_rows(o.reshape(-1, 128), l.reshape(-1), exp_o, exp_l, path)
    finally:
        k[0, 0, s, :] = 0.0


def test_query_side_at_max():
    dev = torch.device("cuda:0")
    hq, nq, nk = 8, NQ_MAX, 64
    say(f"max-size query side: Hq={hq} Nq={nq} Nk={nk}, Q and O {hq * nq * 128 * 2 / 2**30:.2f} GiB each")
    flat = torch.arange(hq * nq, device=dev, dtype=torch.int64)
    a = ((flat >> 18) & 7).to(torch.float32)                 # [hq * nq]
    q = (a / 64.0).to(torch.bfloat16).view(1, hq, nq, 1).expand(1, hq, nq, 128).contiguous()
    del flat
    k = torch.zeros((1, hq, nk, 128), dtype=torch.bfloat16, device=dev)
    k[:, :, 0, :] = 1.0
    kidx = torch.arange(nk, device=dev, dtype=torch.float32)
    vrow = (torch.remainder(kidx, 16) - 7.5) / 16.0
    v = vrow.view(1, 1, nk, 1).expand(1, hq, nk, 128).to(torch.bfloat16).contiguous()
    out = torch.full((1, hq, nq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((1, hq, nq), float("nan"), dtype=torch.float32, device=dev)
    o, l = fwd(q, k, v, causal=False, scale=1.0, out=out, lse=lse)
    torch.cuda.synchronize()
    # closed forms per value of a, as a table indexed on the GPU
    vk = [((kk % 16) - 7.5) / 16.0 for kk in range(nk)]
    rest = sum(vk[1:])
    tab_o = torch.tensor([(math.exp(2 * aa) * vk[0] + rest) / (math.exp(2 * aa) + nk - 1) for aa in range(8)],
                         dtype=torch.float64, device=dev)
    tab_l = torch.tensor([math.log(math.exp(2 * aa) + nk - 1) for aa in range(8)], dtype=torch.float64, device=dev)
    ai = a.to(torch.int64)
    exp_l = tab_l[ai]
    lerr = float((l.reshape(-1).double() - exp_l).abs().max())
    assert torch.isfinite(l).all(), "non-finite LSE"
    worst = 0.0
    o2 = o.view(-1, 128)
    for r0 in range(0, o2.shape[0], 1 << 20):                # 1M rows at a time
        blk = o2[r0:r0 + (1 << 20)].double()
        assert torch.isfinite(blk).all(), f"non-finite O in rows {r0}.."
        worst = max(worst, float((blk - tab_o[ai[r0:r0 + (1 << 20)]][:, None]).abs().max()))
    say(f"  query side: max|dO| = {worst:.3e}, max|dLSE| = {lerr:.3e} over {o2.shape[0]} rows")
    assert worst <= BF16_MAX_ABS and lerr <= LSE_MAX_ABS


def test_backward_key_side_at_max(key_side):
    """fa_bwd over the 2^24 - 1 keys (Nq = 64, causal): with dO = 1/64 in every
    element, dV[s] = P_s * sum_i dO[i] = P_s per column (P_s = e^30 / Z, Z as
    above), every other dV row is 64 P_0 / 64 = 1 / Z (about 1e-13), and dQ and
    dK are of the order 1 - P_s (about 1e-6): all within the bf16 bounds of zero."""
    from exact_attention_105_amd import bwd
    k, v = key_side
    dev = k.device
    s = NK_MAX - 100
    k[0, 0, s, :] = 1.0
    try:
        nq = 64
        q = torch.full((1, 1, nq, 128), SPIKE_SCORE / 128.0, dtype=torch.bfloat16, device=dev)
        say(f"max-size backward: Nq={nq} Nk={NK_MAX} causal")
        o, l = fwd(q, k, v, causal=True, scale=1.0)
        do = torch.full_like(q, 1.0 / 64.0)
        dq = torch.full_like(q, float("nan"))
        dk = torch.full_like(k, float("nan"))
        dv = torch.full_like(v, float("nan"))
        bwd(q, k, v, o, l, do, causal=True, scale=1.0, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert bool(torch.isfinite(t).all()), f"{name} not finite (unwritten rows stay NaN)"
        # rows see keys up to Nk - 64 + i: Z differs per row, P_s = e^30 / Z_i
        ps = [math.exp(SPIKE_SCORE) / (math.exp(SPIKE_SCORE) + (NK_MAX - nq + i + 1) - 1) for i in range(nq)]
        want_dvs = sum(ps) / 64.0
        got = dv[0, 0, s].float()
        err_s = float((got - want_dvs).abs().max())
        others = float(dv[0, 0, torch.tensor([0, 1 << 23, NK_MAX - 200, NK_MAX - 1], device=dev)].float().abs().max())
        dq_max = float(dq.float().abs().max())
        dk_max = float(dk.float().abs().max())
        say(f"  dV[spike] error {err_s:.3e} (value {want_dvs:.6f}); max |dV| elsewhere {others:.3e}; "
            f"max |dQ| {dq_max:.3e}; max |dK| {dk_max:.3e}")
        assert err_s <= BF16_MAX_ABS and others <= BF16_MAX_ABS and dq_max <= BF16_MAX_ABS and dk_max <= BF16_MAX_ABS
    finally:
        k[0, 0, s, :] = 0.0
