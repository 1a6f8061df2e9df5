"""The Python binding refuses output, statistics and workspace tensors that
the library could not write safely (wrong shape, dtype, layout or device)
before any call into the library, for every entry point that takes them."""
import pytest
import torch

import exact_attention_105_amd as fa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    fa.load()
    return torch.device("cuda:0")


def _qkv(dev, B=1, Hq=2, Hkv=2, Nq=40, Nk=70, d=128):
    g = torch.Generator(device="cpu").manual_seed(7)
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(dev)
    return mk(B, Hq, Nq, d), mk(B, Hkv, Nk, d), mk(B, Hkv, Nk, d)


def test_fwd_refuses_bad_outputs(dev):
    q, k, v = _qkv(dev)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, out=torch.empty((1, 2, 40, 128), dtype=torch.bfloat16))           # host memory
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, lse=torch.empty((1, 2, 80), dtype=torch.float32, device=dev)[:, :, ::2])  # strided
    o, lse = fa.fwd(q, k, v)                                                           # and the good call runs
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_splitkv_refuses_bad_outputs_and_workspace(dev):
    q, k, v = _qkv(dev, B=2, Hq=8, Hkv=2, Nq=1, Nk=5000)
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, n_splits=4, out=torch.empty((2, 8, 1, 64), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, n_splits=4, lse=torch.empty((2, 8, 1), dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, n_splits=4, workspace=torch.empty(10, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, n_splits=4, workspace=torch.empty(4 * 2 * 8 * 129, dtype=torch.float32))
    o, lse = fa.fwd_splitkv(q, k, v, n_splits=4)
    ref_o, ref_lse = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    assert (o.float() - ref_o.float()).abs().max().item() < 2e-2
    assert (lse - ref_lse).abs().max().item() < 1e-3


def test_bwd_refuses_bad_gradients_and_workspace(dev):
    q, k, v = _qkv(dev, Nq=64, Nk=64)
    o, lse = fa.fwd(q, k, v, causal=True)
    do = torch.ones_like(o)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=torch.empty_like(q).cpu())
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, do, causal=True, workspace=torch.empty(2 * 2 * 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, do, causal=True, workspace=torch.empty(8, dtype=torch.float32, device=dev))


def test_rotate_refuses_bad_scale_and_work(dev):
    x = torch.randn(64, 128, device=dev)
    with pytest.raises(ValueError):
        fa.rotate_quantize(x, scale=torch.empty(0, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        fa.rotate_quantize(x, work=torch.empty(1, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        fa.rotate_quantize(x, scale=torch.empty(1, dtype=torch.float32))
    codes, scale = fa.rotate_quantize(x)
    torch.cuda.synchronize()
    assert scale.item() > 0
