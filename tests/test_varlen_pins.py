"""Pins of the variable-length oracle (oracle.attention_varlen): it must
reduce to the batch definition, which the attention oracle's own pins fix.

* one sequence equals the [1, H, N, d] batch of the same tokens;
* equal-length sequences equal the batch with B = number of sequences;
* sequences are independent: adding, removing or reordering other sequences
  does not change a sequence's rows;
* per-sequence Nq != Nk follows the bottom-right causal alignment of that
  sequence alone; empty sequences produce no rows.
"""
import numpy as np

import oracle
from synth.inputs import f32_to_bf16_bits


def packed(total, H, d, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((total, H, d)).astype(np.float32))


def to_batch(x, cu, s):
    return np.ascontiguousarray(x[cu[s]:cu[s + 1]].transpose(1, 0, 2)[None])


def test_single_sequence_is_the_batch_problem():
    q, k, v = packed(37, 4, 16, 1), packed(53, 2, 16, 2), packed(53, 2, 16, 3)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, [0, 37], [0, 53], causal=causal, scale=0.3)
        ob, lb = oracle.attention(to_batch(q, [0, 37], 0), to_batch(k, [0, 53], 0), to_batch(v, [0, 53], 0),
                                  causal=causal, scale=0.3)
        assert np.array_equal(o, ob[0].transpose(1, 0, 2)) and np.array_equal(lse, lb[0])


def test_equal_lengths_are_a_batch():
    n, N, H, d = 3, 20, 2, 8
    q, k, v = packed(n * N, H, d, 4), packed(n * N, H, d, 5), packed(n * N, H, d, 6)
    cu = [i * N for i in range(n + 1)]
    o, lse = oracle.attention_varlen(q, k, v, cu, cu, causal=True, scale=0.4)
    qb = np.ascontiguousarray(q.reshape(n, N, H, d).transpose(0, 2, 1, 3))
    kb = np.ascontiguousarray(k.reshape(n, N, H, d).transpose(0, 2, 1, 3))
    vb = np.ascontiguousarray(v.reshape(n, N, H, d).transpose(0, 2, 1, 3))
    ob, lb = oracle.attention(qb, kb, vb, causal=True, scale=0.4)
    assert np.array_equal(o, ob.transpose(0, 2, 1, 3).reshape(n * N, H, d))
    assert np.array_equal(lse, lb.transpose(1, 0, 2).reshape(H, n * N))


def test_sequences_are_independent_and_follow_their_own_alignment():
    H, Hkv, d = 4, 2, 8
    lq, lk = [5, 0, 9, 3], [7, 4, 2, 3]          # Nq > Nk, Nq < Nk, an empty query side
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = packed(cq[-1], H, d, 7), packed(ck[-1], Hkv, d, 8), packed(ck[-1], Hkv, d, 9)
    o, lse = oracle.attention_varlen(q, k, v, cq, ck, causal=True, scale=0.5)
    for s in range(len(lq)):
        if lq[s] == 0:
            continue
        ob, lb = oracle.attention(to_batch(q, cq, s), to_batch(k, ck, s), to_batch(v, ck, s),
                                  causal=True, scale=0.5)
        assert np.array_equal(o[cq[s]:cq[s + 1]], ob[0].transpose(1, 0, 2))
        assert np.array_equal(lse[:, cq[s]:cq[s + 1]], lb[0])
    # sequence 2 sees keys 0..1 of its own only: Nq=9 > Nk=2, so its first 7 rows see nothing
    assert np.all(np.isneginf(lse[:, cq[2]:cq[2] + 7])) and np.all(np.isfinite(lse[:, cq[2] + 7:cq[3]]))
    # reordering the sequences permutes the rows and nothing else
    order = [3, 0, 2, 1]
    q2 = np.concatenate([q[cq[s]:cq[s + 1]] for s in order])
    k2 = np.concatenate([k[ck[s]:ck[s + 1]] for s in order])
    v2 = np.concatenate([v[ck[s]:ck[s + 1]] for s in order])
    cq2 = np.concatenate([[0], np.cumsum([lq[s] for s in order])])
    ck2 = np.concatenate([[0], np.cumsum([lk[s] for s in order])])
    o2, _ = oracle.attention_varlen(q2, k2, v2, cq2, ck2, causal=True, scale=0.5)
    assert np.array_equal(o2, np.concatenate([o[cq[s]:cq[s + 1]] for s in order]))


def test_backward_reduces_to_the_batch_problem():
    """The packed backward oracle: one sequence equals the batch backward of
    the same tokens; sequences are independent (another sequence's tokens do
    not change them); an empty side gives zero gradients."""
    H, Hkv, d = 4, 2, 8
    lq, lk = [6, 0, 9], [7, 3, 2]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = packed(cq[-1], H, d, 11), packed(ck[-1], Hkv, d, 12), packed(ck[-1], Hkv, d, 13)
    do = packed(cq[-1], H, d, 14)
    dq, dk, dv = oracle.attention_bwd_varlen(q, k, v, do, cq, ck, causal=True, scale=0.5)
    for s in (0, 2):
        gq, gk, gv = oracle.attention_bwd(to_batch(q, cq, s), to_batch(k, ck, s), to_batch(v, ck, s),
                                          to_batch(do, cq, s), causal=True, scale=0.5)
        assert np.array_equal(dq[cq[s]:cq[s + 1]], gq[0].transpose(1, 0, 2))
        assert np.array_equal(dk[ck[s]:ck[s + 1]], gk[0].transpose(1, 0, 2))
        assert np.array_equal(dv[ck[s]:ck[s + 1]], gv[0].transpose(1, 0, 2))
    assert not dk[ck[1]:ck[2]].any() and not dv[ck[1]:ck[2]].any()      # keys no query reads
