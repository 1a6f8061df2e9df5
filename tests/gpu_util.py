"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI (via the ctypes binding), and compare with the
oracle under the stated tolerances.

Tolerances (bf16 path): max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3
over the compared elements, with O the GPU's bfloat16 output widened to
float64 and O_ref the fp64 oracle on the same bfloat16 inputs; LSE max abs
<= 1e-3.  FP8 path: relative RMSE ||O - O_ref|| / ||O_ref|| <= 5e-2 against
the oracle on the dequantised E4M3 inputs; LSE within the per-row bound of
fp8_lse_bound (the matrix instruction's accumulation error plus 1e-3).
These bounds are the project's stated acceptance bounds; the pages print
none.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from exact_attention_105_amd import fwd

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
FP8_RRMSE = 5e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: dict, dtype: str):
    dev = torch.device("cuda:0")
    if dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(torch.float8_e4m3fn)
    return conv(x["q"]), conv(x["k"]), conv(x["v"])


def run_gpu(x: dict, dtype: str, causal: bool, scale: float, poison: bool = True):
    """Run the HIP path; returns (O float64 numpy, LSE float64 numpy)."""
    q, k, v = to_device(x, dtype)
    B, Hq, Nq, d = q.shape
    out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if poison:                       # unwritten elements would show up as NaN
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    o, l = fwd(q, k, v, causal=causal, scale=scale, descale=x.get("descale"), out=out, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), l.cpu().double().numpy()


def compare_bf16(o, lse, o_ref, lse_ref, what: str):
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf_ref), f"{what}: -inf LSE pattern differs"
    err = np.abs(o - o_ref)
    worst = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    lerr = np.abs(np.where(ninf_ref, 0.0, lse - np.where(ninf_ref, 0.0, lse_ref)))
    lworst = float(lerr.max()) if lerr.size else 0.0
    loc = np.unravel_index(int(err.argmax()), err.shape) if err.size else ()
    say(f"  {what}: max|dO|={worst:.3e} at {loc} (|O_ref|={abs(float(o_ref[loc])) if err.size else 0:.3f}) "
        f"mean|dO|={mean:.3e} max|dLSE|={lworst:.3e}")
    assert worst <= BF16_MAX_ABS, f"{what}: max abs error {worst} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean abs error {mean} > {BF16_MEAN_ABS}"
    assert lworst <= LSE_MAX_ABS, f"{what}: LSE error {lworst} > {LSE_MAX_ABS}"
    return worst, mean, lworst


# The fp8 matrix instruction (v_mfma ... f8f6f4) adds its 64 products in
# chunks of 8, each product aligned to the largest exponent in its chunk and
# truncated there (measured on the GPU by the microbenchmark
# exact_attention_105_amd/microbench/fp8_accumulation.hip): a score's error is at
# most FP8_MFMA_TRUNC * sum_t |q_t k_t| (the measured worst case is about half
# of that).  A row's log-sum-exp moves by at most the largest error of its
# scores, so the LSE bound of an FP8 row is FP8_MFMA_TRUNC * |scale| *
# max_j sum_t |q_t k_jt| on top of the bf16 path's LSE tolerance.
FP8_MFMA_TRUNC = 2.0 ** -10


def fp8_lse_bound(x, rows, scale):
    """Per-row LSE bound for the FP8 path on the listed flat rows (or all rows)."""
    sq, sk, _ = x["descale"]
    q = oracle.decode(x["q"], "e4m3", sq)        # [B, Hq, Nq, d] float64
    k = oracle.decode(x["k"], "e4m3", sk)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    if rows is None:
        rows = np.arange(B * Hq * Nq)
    rows = np.asarray(rows)
    out = np.empty(rows.size)
    head = rows // Nq
    for hf in np.unique(head):
        b, h = divmod(int(hf), Hq)
        sel = np.nonzero(head == hf)[0]
        qa = np.abs(q[b, h, rows[sel] % Nq]).astype(np.float32)
        ka = np.abs(k[b, h // (Hq // Hkv)]).astype(np.float32)
        mx = np.zeros(sel.size, dtype=np.float64)
        for c in range(0, ka.shape[0], 4096):
            mx = np.maximum(mx, (qa @ ka[c:c + 4096].T).max(axis=1))
        out[sel] = FP8_MFMA_TRUNC * abs(scale) * mx * 1.001 + LSE_MAX_ABS
    return out


def compare_fp8(o, lse, o_ref, lse_ref, what: str, lse_bound=None):
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    rrmse = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    ninf = np.isneginf(lse_ref)
    lerr = np.abs(np.where(ninf, 0.0, lse - np.where(ninf, 0.0, lse_ref))).reshape(-1)
    lworst = float(lerr.max()) if lse.size else 0.0
    msg = ""
    if lse_bound is not None and lse.size:
        ratio = lerr / np.asarray(lse_bound).reshape(-1)
        msg = f" (max |dLSE| / row bound = {float(ratio.max()):.3f})"
        assert np.all(ratio <= 1.0), f"{what}: LSE error above the FP8 accumulation bound (worst ratio {ratio.max()})"
    say(f"  {what}: rRMSE={rrmse:.3e} max|dLSE|={lworst:.3e}{msg}")
    assert rrmse <= FP8_RRMSE, f"{what}: rRMSE {rrmse} > {FP8_RRMSE}"
    return rrmse, lworst


def sample_rows(B, Hq, Nq, seed=0, per_head=24, heads=None):
    """Flat row indices (b*Hq + h)*Nq + i covering edges, tile boundaries and random rows."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, Nq // 2, Nq - 2, Nq - 1}
    fixed = sorted(i for i in fixed if 0 <= i < Nq)
    rows = []
    all_heads = [(b, h) for b in range(B) for h in range(Hq)]
    if heads is None:
        pick = {0, len(all_heads) - 1}
        pick.update(rng.choice(len(all_heads), size=min(6, len(all_heads)), replace=False).tolist())
        heads = [all_heads[i] for i in sorted(pick)]
    for (b, h) in heads:
        extra = rng.choice(Nq, size=min(per_head, Nq), replace=False).tolist() if Nq > 0 else []
        for i in sorted(set(fixed) | set(extra)):
            rows.append((b * Hq + h) * Nq + i)
    return np.array(sorted(set(rows)), dtype=np.int64)


def head_rows(Hq, Nq, heads):
    """Flat row indices (b*Hq + h)*Nq + i of every row of the listed (b, h) heads."""
    return np.concatenate([np.arange((b * Hq + h) * Nq, (b * Hq + h + 1) * Nq, dtype=np.int64)
                           for (b, h) in heads])


def complete_heads(B, Hq, Hkv):
    """The (b, h) heads a full-size parity test compares row for row: the first
    head of the first key/value group, the last head of that group (when heads
    share keys), and the last head of the last batch entry."""
    g = Hq // Hkv
    heads = [(0, 0)]
    if g > 1:
        heads.append((0, g - 1))
    heads.append((B - 1, Hq - 1))
    return sorted(set(heads))


def oracle_ref(x, dtype, causal, scale, rows=None):
    return oracle.attention(x["q"], x["k"], x["v"], causal=causal, scale=scale,
                            dtype=dtype, descale=x.get("descale"), rows=rows)
