"""PyTorch-facing wrappers of the attention library.

PyTorch provides device memory and the current HIP stream; the computation
is entirely the HIP library's (``fa_fwd``, ``fa_bwd`` and
``fa_rotate_quantize_e4m3`` in include/fa.h).
"""
from __future__ import annotations

import math

import torch

from . import _lib

_FP8_TYPES = (torch.uint8, torch.float8_e4m3fn)


def _on_device(dev, **tensors):
    """Every given tensor (None is skipped) is a contiguous GPU tensor on
    ``dev``: the library writes through raw pointers, so a tensor elsewhere,
    or a strided view, must be refused before the call."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"{name} must be a GPU tensor on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


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
    _on_device(q.device, out=out, lse=lse)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                     lse.data_ptr() if lse is not None else None,
                     B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale, dtype, descale, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return out, lse


def default_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int) -> int:
    """A split count that gives the decode grid about 128 workgroups while
    keeping at least 4096 keys per split (measured on a 64K-key, 8-head
    decode: 16 splits stream K and V at 5.1 TB/s; more, shorter splits lose
    to per-workgroup set-up and the extra rounds of workgroups)."""
    units = B * Hkv * ((Nq * (Hq // Hkv) + 31) // 32)
    return int(max(1, min(256, -(-128 // max(units, 1)), Nk // 4096)))


def _splitkv_args(q, k, v, causal, scale, n_splits, out, lse):
    """Checks and defaults shared by fwd_splitkv and fwd_splitkv_noalloc."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 [B, H, N, d] GPU tensor")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if Bk != B or dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = default_splits(B, Hq, Hkv, Nq, Nk)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, Hq, Nq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [B, Hq, Nq, d] tensor")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    return (B, Hq, Hkv, Nq, Nk, d), float(scale), int(n_splits), out, lse


def fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                scale: float | None = None, n_splits: int | None = None, workspace: torch.Tensor | None = None,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Decode-shaped attention (bf16, d = 128, Nq <= 16) with the keys split
    over ``n_splits`` workgroups per key/value head and merged afterwards;
    returns (O, LSE) like ``fwd``.  ``n_splits`` defaults to
    ``default_splits``; ``workspace`` holds n_splits*B*Hq*Nq*(d+1) floats."""
    dims, scale, n_splits, out, lse = _splitkv_args(q, k, v, causal, scale, n_splits, out, lse)
    B, Hq, Hkv, Nq, Nk, d = dims
    need = n_splits * B * Hq * Nq * (d + 1)
    if workspace is None and n_splits > 1:
        workspace = torch.empty(max(need, 1), dtype=torch.float32, device=q.device)
    elif workspace is not None and (workspace.dtype != torch.float32 or workspace.numel() < need):
        raise ValueError(f"workspace must hold {need} float32 values")
    _on_device(q.device, k=k, v=v, out=out, lse=lse, workspace=workspace)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale, _lib.FA_DTYPE_BF16, n_splits,
                             workspace.data_ptr() if workspace is not None else None, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return out, lse


def fwd_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, out: torch.Tensor,
                        lse: torch.Tensor, causal: bool = False, scale: float | None = None,
                        n_splits: int | None = None):
    """``fwd_splitkv`` without a workspace: the split partials go to the
    library's own scratch array on each GPU (``_lib.SPLITKV_SCRATCH_FLOATS``
    floats; larger problems raise FaError).  The caller passes ``out`` and
    ``lse``, so the call allocates nothing.  Calls that overlap on one GPU
    share that array and race: order them on one stream."""
    dims, scale, n_splits, out, lse = _splitkv_args(q, k, v, causal, scale, n_splits, out, lse)
    B, Hq, Hkv, Nq, Nk, d = dims
    _on_device(q.device, k=k, v=v, out=out, lse=lse)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale, _lib.FA_DTYPE_BF16,
                                     n_splits, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return out, lse


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, max_seqlen_q: int, *, causal: bool = False,
               scale: float | None = None, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Exact attention over a packed batch of variable-length sequences.

    q [total_q, Hq, d], k and v [total_k, Hkv, d] (bfloat16, contiguous, one
    GPU); cu_seqlens_q / cu_seqlens_k int32 GPU tensors of n_seqs + 1
    offsets; max_seqlen_q at least every query length.  Returns (O
    [total_q, Hq, d] bfloat16, LSE [Hq, total_q] float32).  Runs on torch's
    current stream.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dim() != 3 or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 [tokens, H, d] GPU tensor")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU vector")
    n_seqs = cu_seqlens_q.numel() - 1
    if n_seqs < 0 or cu_seqlens_k.numel() != n_seqs + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold n_seqs + 1 offsets")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk_ = k.shape
    if dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((total_q, Hq, d), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (total_q, Hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [total_q, Hq, d] tensor")
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Hq, total_q] tensor")
    _on_device(q.device, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, out=out, lse=lse)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), n_seqs, int(max_seqlen_q),
                            total_q, total_k, Hq, Hkv, d, int(bool(causal)), scale, _lib.FA_DTYPE_BF16, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return out, lse


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, causal: bool = False, scale: float | None = None,
        dq: torch.Tensor | None = None, dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
        workspace: torch.Tensor | None = None):
    """Exact attention backward: returns (dQ, dK, dV), bfloat16.

    q, k, v, ``causal`` and ``scale`` as given to ``fwd``; o and lse are the
    outputs ``fwd`` returned for them, dout the gradient of the loss with
    respect to o (bfloat16, o's shape).  ``workspace`` holds 2*B*Hq*Nq
    floats.  Runs on torch's current stream.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 [B, H, N, d] GPU tensor")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if Bk != B or dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def out_like(t, ref, name):
        if t is None:
            return torch.empty(ref.shape, dtype=torch.bfloat16, device=ref.device)
        if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(ref.shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor shaped like {tuple(ref.shape)}")
        return t

    dq, dk, dv = out_like(dq, q, "dq"), out_like(dk, k, "dk"), out_like(dv, v, "dv")
    if workspace is None:
        workspace = torch.empty(max(2 * B * Hq * Nq, 1), dtype=torch.float32, device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < 2 * B * Hq * Nq:
        raise ValueError("workspace must hold 2*B*Hq*Nq float32 values")
    _on_device(q.device, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, workspace=workspace)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                     B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale, _lib.FA_DTYPE_BF16, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return dq, dk, dv


def bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
               dout: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
               max_seqlen_k: int, *, causal: bool = False, scale: float | None = None,
               dq: torch.Tensor | None = None, dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None):
    """Backward of ``fwd_varlen``: returns (dQ, dK, dV) in the packed layouts.

    o and lse [Hq, total_q] are what ``fwd_varlen`` returned; dout is the
    gradient of the loss with respect to o.  ``workspace`` holds
    2*Hq*total_q floats.  Runs on torch's current stream.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not t.is_cuda or t.dim() != 3 or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 [tokens, H, d] GPU tensor")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU vector")
    n_seqs = cu_seqlens_q.numel() - 1
    if n_seqs < 0 or cu_seqlens_k.numel() != n_seqs + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold n_seqs + 1 offsets")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk_ = k.shape
    if dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [Hq, total_q] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def out_like(t, ref, name):
        if t is None:
            return torch.empty(ref.shape, dtype=torch.bfloat16, device=ref.device)
        if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(ref.shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor shaped like {tuple(ref.shape)}")
        return t

    dq, dk, dv = out_like(dq, q, "dq"), out_like(dk, k, "dk"), out_like(dv, v, "dv")
    if workspace is None:
        workspace = torch.empty(max(2 * Hq * total_q, 1), dtype=torch.float32, device=q.device)
    elif workspace.dtype != torch.float32 or workspace.numel() < 2 * Hq * total_q:
        raise ValueError("workspace must hold 2*Hq*total_q float32 values")
    _on_device(q.device, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, workspace=workspace,
               cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = _lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), n_seqs, int(max_seqlen_q),
                            int(max_seqlen_k), total_q, total_k, Hq, Hkv, d, int(bool(causal)), scale,
                            _lib.FA_DTYPE_BF16, stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return dq, dk, dv


def sign_bits(signs) -> list:
    """Pack a length-d sequence of +-1 (or booleans, True = negate) into the
    d/32 words fa_rotate_quantize_e4m3 takes."""
    words = [0] * ((len(signs) + 31) // 32)
    for j, sgn in enumerate(signs):
        neg = bool(sgn) if isinstance(sgn, (bool,)) else float(sgn) < 0
        if neg:
            words[j >> 5] |= 1 << (j & 31)
    return words


def rotate_quantize(x: torch.Tensor, *, rotate: bool = True, signs=None,
                    codes: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                    work: torch.Tensor | None = None):
    """Incoherent processing before FP8 attention: returns (codes, scale).

    x: contiguous bfloat16 or float32 GPU tensor whose last dimension d is 64
    or 128.  Every row is multiplied by M = D H / sqrt(d) (D = diag(signs),
    H Sylvester-Hadamard; skipped when ``rotate`` is False) and the result is
    quantised per tensor to E4M3: codes (torch.float8_e4m3fn, x's shape) and
    a one-element float32 tensor s = max|x M| / 448.  Rotate Q and K with the
    same ``signs`` (a length-d sequence of +-1); quantise V without rotation.
    Runs on torch's current stream; ``work`` is a one-float workspace.
    """
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    if x.dtype == torch.bfloat16:
        xd = _lib.FA_DTYPE_BF16
    elif x.dtype == torch.float32:
        xd = _lib.FA_DTYPE_F32
    else:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    d = x.shape[-1] if x.dim() else 0
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    elif codes.shape != x.shape or codes.dtype not in _FP8_TYPES or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous float8_e4m3fn/uint8 tensor shaped like x")
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    elif scale.dtype != torch.float32 or scale.numel() < 1:
        raise ValueError("scale must be a float32 tensor of at least one element")
    if work is None:
        work = torch.empty(1, dtype=torch.float32, device=x.device)
    elif work.dtype != torch.float32 or work.numel() < 1:
        raise ValueError("work must be a float32 tensor of at least one element")
    _on_device(x.device, codes=codes, scale=scale, work=work)
    if signs is not None and len(signs) != d:
        raise ValueError("signs must have one entry per feature")
    bits = sign_bits(signs) if signs is not None else None
    stream = torch.cuda.current_stream(x.device).cuda_stream
    st = _lib.fa_rotate_quantize_e4m3(x.data_ptr(), xd, rows, d, int(bool(rotate)), bits,
                                      codes.data_ptr(), scale.data_ptr(), work.data_ptr(), stream)
    if st != _lib.FA_SUCCESS:
        raise _lib.FaError(st, _lib.status_string(st))
    return codes, scale
