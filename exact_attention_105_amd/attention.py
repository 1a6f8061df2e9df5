"""PyTorch-facing wrapper of the attention forward pass.

PyTorch provides device memory and the current HIP stream; the computation
is entirely the HIP library's (``fa_fwd`` in include/fa.h).
"""
from __future__ import annotations

import math

import torch

from . import _lib

_FP8_TYPES = (torch.uint8, torch.float8_e4m3fn)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        scale: float | None = None, descale=None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, return_lse: bool = True):
    """Exact attention forward: returns (O, LSE).

    q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d], contiguous, on one GPU.
    bfloat16 inputs, or FP8 E4M3 codes (torch.float8_e4m3fn or uint8) with
    ``descale=(sq, sk, sv)``.  O is bfloat16 [B, Hq, Nq, d]; LSE float32
    [B, Hq, Nq] (natural log).  ``scale`` defaults to 1/sqrt(d).  Causal
    masking is bottom-right aligned (key j visible to query i iff
    j <= i + Nk - Nq).  Runs on torch's current stream.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if q.dtype == torch.bfloat16 and k.dtype == v.dtype == torch.bfloat16:
        dtype = _lib.FA_DTYPE_BF16
        if descale is not None:
            raise ValueError("descale is only for FP8 inputs")
    elif q.dtype in _FP8_TYPES and k.dtype in _FP8_TYPES and v.dtype in _FP8_TYPES:
        dtype = _lib.FA_DTYPE_FP8_E4M3
        if descale is None:
            raise ValueError("FP8 inputs need descale=(sq, sk, sv)")
    else:
        raise TypeError(f"unsupported dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, Hq, Nq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [B, Hq, Nq, d] tensor")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                     lse.data_ptr() if lse is not None else None,
                     B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale, dtype, descale, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return out, lse
