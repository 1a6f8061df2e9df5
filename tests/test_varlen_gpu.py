"""GPU parity of fa_fwd_varlen (packed batches of sequences of different
lengths) against the oracle, which runs every sequence as its own batch
problem.  Same tolerances as the fixed-length bf16 path (gpu_util.py)."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_105_amd import fwd, fwd_varlen
from gpu_util import compare_bf16, say
from synth.inputs import VARLEN_WORKLOADS, make_varlen_inputs, workload_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_105_amd as fa
    fa.load()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def run_varlen(x, causal, scale, max_q=None):
    q, k, v = (dev_bf16(x[n]) for n in ("q", "k", "v"))
    cq = torch.from_numpy(x["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(x["cu_k"]).to("cuda:0")
    lens = np.diff(x["cu_q"])
    max_q = int(lens.max()) if max_q is None and lens.size else (max_q or 0)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((q.shape[1], q.shape[0]), float("nan"), dtype=torch.float32, device=q.device)
    o, l = fwd_varlen(q, k, v, cq, ck, max_q, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), l.cpu().double().numpy()


# (query lengths, key lengths or None for the same, Hq, Hkv, d, causal)
CASES = [
    ([128, 1, 300, 0, 129], None, 4, 2, 128, True),
    ([128, 1, 300, 0, 129], None, 4, 4, 64, False),
    ([77, 256, 5], [200, 100, 5], 2, 1, 128, True),      # Nq < Nk, Nq > Nk, Nq = Nk per sequence
    ([77, 256, 5], [200, 100, 5], 2, 2, 64, True),
    ([500, 3, 260], [1, 700, 0], 4, 2, 128, False),       # a single key, an empty key side
    ([1000], None, 8, 2, 128, True),
    # more sequences than a wave has lanes (the grid's slot search spans several 64-sequence chunks),
    # lengths from 0 to 400 with empty and one-row sequences among them
    (np.random.default_rng(150).integers(0, 401, 150).tolist(), None, 2, 1, 64, True),
    (np.random.default_rng(70).integers(0, 300, 70).tolist(), None, 2, 2, 128, False),
    # padded grids 8x or more the tiles that exist: these take the compact grid (one slot per tile,
    # found by a search over the sequences' tile counts), with 2 and 5 chunks of 64 sequences
    ([2000] + [10] * 100, None, 2, 1, 128, True),
    ([3000] + np.random.default_rng(300).integers(0, 21, 299).tolist(), None, 2, 2, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[(f"{c[0]}" if len(c[0]) <= 8 else f"{len(c[0])}seqs")
                                             + f"x{c[1]}H{c[2]}/{c[3]}d{c[4]}{'c' if c[5] else ''}" for c in CASES])
def test_varlen_matches_oracle(case):
    lq, lk, Hq, Hkv, d, causal = case
    lk = lq if lk is None else lk
    x = make_varlen_inputs(np.array(lq), np.array(lk), Hq, Hkv, d, 4242 + sum(lq))
    scale = 1.0 / math.sqrt(d)
    say(f"varlen {case}")
    o, lse = run_varlen(x, causal, scale)
    o_ref, lse_ref = oracle.attention_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], causal=causal, scale=scale)
    compare_bf16(o, lse, o_ref, lse_ref, f"varlen {case}")


def test_equal_lengths_match_the_batch_kernel_bit_for_bit():
    """The packed path and the [B, H, N, d] path run the same arithmetic."""
    n, N, Hq, Hkv, d = 3, 300, 4, 2, 128
    x = make_varlen_inputs(np.full(n, N), np.full(n, N), Hq, Hkv, d, 77)
    for causal in (False, True):
        o, lse = run_varlen(x, causal, 0.09)
        qb = dev_bf16(np.ascontiguousarray(x["q"].reshape(n, N, Hq, d).transpose(0, 2, 1, 3)))
        kb = dev_bf16(np.ascontiguousarray(x["k"].reshape(n, N, Hkv, d).transpose(0, 2, 1, 3)))
        vb = dev_bf16(np.ascontiguousarray(x["v"].reshape(n, N, Hkv, d).transpose(0, 2, 1, 3)))
        ob, lb = fwd(qb, kb, vb, causal=causal, scale=0.09)
        torch.cuda.synchronize()
        ob = ob.float().cpu().double().numpy().transpose(0, 2, 1, 3).reshape(n * N, Hq, d)
        lb = lb.cpu().double().numpy().transpose(1, 0, 2).reshape(Hq, n * N)
        say(f"  equal lengths causal={causal}: max |varlen - batch| O {np.abs(o - ob).max():.1e} LSE {np.abs(lse - lb).max():.1e}")
        assert np.array_equal(o, ob) and np.array_equal(lse, lb)


@pytest.mark.parametrize("name", ["varlen_mix", "varlen_skew"])
def test_varlen_workload_sampled_rows(name):
    """The ragged bench workloads at full size (varlen_skew takes the compact
    grid): sampled rows of every sequence against the oracle on that
    sequence."""
    w = VARLEN_WORKLOADS[name]
    lens = workload_lengths(w)
    x = make_varlen_inputs(lens, lens, w["Hq"], w["Hkv"], w["d"], w["seed"])
    scale = 1.0 / math.sqrt(w["d"])
    say(f"{name}: {len(lens)} sequences, {int(lens.sum())} tokens")
    o, lse = run_varlen(x, w["causal"], scale)
    rng = np.random.default_rng(3)
    cu = x["cu_q"]
    for s in range(len(lens)):
        L = int(lens[s])
        qs = np.ascontiguousarray(x["q"][cu[s]:cu[s + 1]].transpose(1, 0, 2)[None])
        ks = np.ascontiguousarray(x["k"][cu[s]:cu[s + 1]].transpose(1, 0, 2)[None])
        vs = np.ascontiguousarray(x["v"][cu[s]:cu[s + 1]].transpose(1, 0, 2)[None])
        rows = rng.choice(w["Hq"] * L, size=min(16, w["Hq"] * L), replace=False)   # flat (h, i) within the sequence
        o_ref, lse_ref = oracle.attention(qs, ks, vs, causal=w["causal"], scale=scale, rows=rows)
        h, i = rows // L, rows % L
        compare_bf16(o[cu[s] + i, h], lse[h, cu[s] + i], o_ref, lse_ref, f"{name} sequence {s} (len {L})")


def run_varlen_bwd(x, do_bits, causal, scale):
    from exact_attention_105_amd import bwd_varlen
    q, k, v = (dev_bf16(x[t]) for t in ("q", "k", "v"))
    do = dev_bf16(do_bits)
    cq = torch.from_numpy(x["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(x["cu_k"]).to("cuda:0")
    mq = int(np.diff(x["cu_q"]).max()) if len(x["cu_q"]) > 1 else 0
    mk = int(np.diff(x["cu_k"]).max()) if len(x["cu_k"]) > 1 else 0
    o, lse = fwd_varlen(q, k, v, cq, ck, mq, causal=causal, scale=scale)
    outs = [torch.full(t.shape, float("nan"), dtype=torch.bfloat16, device=t.device) for t in (q, k, v)]
    dq, dk, dv = bwd_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, causal=causal, scale=scale,
                            dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    return tuple(t.float().cpu().double().numpy() for t in (dq, dk, dv))


# (query lengths, key lengths or None, Hq, Hkv, d, causal)
BWD_CASES = [
    ([128, 1, 300, 0, 129], None, 4, 2, 128, True),
    ([77, 256, 5], [200, 100, 5], 2, 1, 64, True),
    ([500, 3, 260], [1, 700, 0], 4, 2, 128, False),
    ([300, 300], [300, 300], 8, 2, 128, True),
    # the compact grids of the dK/dV and dQ kernels (padded grids 8x or more the tiles that exist)
    ([2000] + [10] * 100, None, 2, 1, 128, True),
    ([1500] + np.random.default_rng(151).integers(0, 21, 150).tolist(), None, 2, 2, 64, False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[(f"{c[0]}" if len(c[0]) <= 8 else f"{len(c[0])}seqs")
                                                 + f"x{c[1]}H{c[2]}/{c[3]}d{c[4]}{'c' if c[5] else ''}"
                                                 for c in BWD_CASES])
def test_varlen_backward_matches_oracle(case):
    from test_bwd_gpu import compare
    from synth.inputs import f32_to_bf16_bits
    lq, lk, Hq, Hkv, d, causal = case
    lk = lq if lk is None else lk
    x = make_varlen_inputs(np.array(lq), np.array(lk), Hq, Hkv, d, 5151 + sum(lq))
    do_bits = f32_to_bf16_bits(np.random.default_rng(sum(lk)).standard_normal(x["q"].shape).astype(np.float32))
    scale = 1.0 / math.sqrt(d)
    say(f"varlen backward {case}")
    got = run_varlen_bwd(x, do_bits, causal, scale)
    ref = oracle.attention_bwd_varlen(x["q"], x["k"], x["v"], do_bits, x["cu_q"], x["cu_k"], causal=causal,
                                      scale=scale)
    compare(got, ref, f"varlen backward {case}")


def test_varlen_backward_equal_lengths_match_the_batch_kernel_bit_for_bit():
    from exact_attention_105_amd import bwd
    from synth.inputs import f32_to_bf16_bits
    n, N, Hq, Hkv, d = 2, 300, 4, 2, 128
    x = make_varlen_inputs(np.full(n, N), np.full(n, N), Hq, Hkv, d, 78)
    do_bits = f32_to_bf16_bits(np.random.default_rng(1).standard_normal(x["q"].shape).astype(np.float32))
    got = run_varlen_bwd(x, do_bits, True, 0.09)
    tb = lambda a, H: np.ascontiguousarray(a.reshape(n, N, H, d).transpose(0, 2, 1, 3))
    qb, kb, vb, dob = (dev_bf16(tb(x["q"], Hq)), dev_bf16(tb(x["k"], Hkv)), dev_bf16(tb(x["v"], Hkv)),
                       dev_bf16(tb(do_bits, Hq)))
    o, lse = fwd(qb, kb, vb, causal=True, scale=0.09)
    dq, dk, dv = bwd(qb, kb, vb, o, lse, dob, causal=True, scale=0.09)
    torch.cuda.synchronize()
    back = lambda t, H: t.float().cpu().double().numpy().transpose(0, 2, 1, 3).reshape(n * N, H, d)
    for name, g, r in zip(("dQ", "dK", "dV"), got, (back(dq, Hq), back(dk, Hkv), back(dv, Hkv))):
        say(f"  equal lengths backward {name}: max |varlen - batch| {np.abs(g - r).max():.1e}")
        assert np.array_equal(g, r), name
