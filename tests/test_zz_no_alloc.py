"""fa_fwd_splitkv_noalloc (split-KV decode with the library's own scratch
array instead of a workspace argument), called through the C ABI, against
fa_fwd_splitkv with a caller workspace: the same kernels and split counts, so
the outputs must match bit for bit.  Two calls in a row, the second on a
smaller problem, so that a stale partial left in the scratch array by the
first call would show; plus the size limit and the oracle on the second."""
import math

import pytest
import torch

import oracle
from exact_attention_105_amd import _lib
from gpu_util import compare_bf16, say, to_device
from synth.inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.load()


def outputs(q):
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    return out, lse


def call_both(x, causal, n_splits):
    """(O, LSE) of fa_fwd_splitkv with a workspace and of
    fa_fwd_splitkv_noalloc, on the same inputs, as CPU tensors."""
    q, k, v = to_device(x, "bf16")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr())
    ws = torch.empty(n_splits * B * Hq * Nq * (d + 1), dtype=torch.float32, device=q.device)
    o1, l1 = outputs(q)
    st = _lib.fa_fwd_splitkv(*ptrs, o1.data_ptr(), l1.data_ptr(), B, Hq, Hkv, Nq, Nk, d, causal, scale,
                             _lib.FA_DTYPE_BF16, n_splits, ws.data_ptr(), stream)
    assert st == _lib.FA_SUCCESS, _lib.status_string(st)
    o2, l2 = outputs(q)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = _lib.fa_fwd_splitkv_noalloc(*ptrs, o2.data_ptr(), l2.data_ptr(), B, Hq, Hkv, Nq, Nk, d, causal, scale,
                                     _lib.FA_DTYPE_BF16, n_splits, stream)
    assert st == _lib.FA_SUCCESS, _lib.status_string(st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return o1.cpu(), l1.cpu(), o2.cpu(), l2.cpu()


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 32 x 32 query heads over 4096 keys, 16 splits (8.5 MB of partials)
    big = (32, 32, 8, 1, 4096, True, 16)
    # second call: smaller, ragged (3000 keys, Nq = 3), other split count
    small = (2, 8, 2, 3, 3000, True, 5)
    for case in (big, small):
        B, Hq, Hkv, Nq, Nk, causal, ns = case
        assert ns * B * Hq * Nq * 129 <= _lib.SPLITKV_SCRATCH_FLOATS
        say(f"noalloc {case}")
        x = make_inputs(B, Hq, Hkv, Nq, Nk, 128, "bf16", 4100 + Nk + ns)
        o1, l1, o2, l2 = call_both(x, causal, ns)
        assert not torch.isnan(o1.float()).any() and not torch.isnan(l1).any()
        assert torch.equal(o1, o2), f"O differs {case}"
        assert torch.equal(l1, l2), f"LSE differs {case}"
        if case is small:
            o_ref, lse_ref = oracle.attention(x["q"], x["k"], x["v"], causal=causal, scale=1.0 / math.sqrt(128))
            compare_bf16(o2.float().double().numpy(), l2.double().numpy(), o_ref, lse_ref, f"noalloc {case}")


def test_noalloc_rejects_problems_above_the_scratch_size():
    """A call needing more than the scratch array is FA_ERROR_INVALID_VALUE
    before any launch; the outputs stay untouched."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, Nq, Nk, d, ns = 64, 64, 8, 4, 1024, 128, 16       # 33.8M floats of partials
    assert ns * B * Hq * Nq * (d + 1) > _lib.SPLITKV_SCRATCH_FLOATS
    q = torch.zeros((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    o, lse = outputs(q)
    st = _lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                     Hkv, Nq, Nk, d, True, 1.0, _lib.FA_DTYPE_BF16, ns,
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.FA_ERROR_INVALID_VALUE
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
    # the same problem with one split needs no scratch and runs
    st = _lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                     Hkv, Nq, Nk, d, True, 1.0, _lib.FA_DTYPE_BF16, 1,
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.FA_SUCCESS
    assert not torch.isnan(o.float()).any()
