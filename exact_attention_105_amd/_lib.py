"""ctypes binding of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind ``fa_fwd``, ``fa_bwd`` and ``fa_rotate_quantize_e4m3``.  There is no CPU
fallback: if the library is missing or a call fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_DTYPE_BF16 = 0
FA_DTYPE_FP8_E4M3 = 1
FA_DTYPE_F32 = 2

FA_SUCCESS = 0
FA_ERROR_INVALID_VALUE = 1
FA_ERROR_NOT_SUPPORTED = 2
FA_ERROR_LAUNCH_FAILURE = 3
SPLITKV_SCRATCH_FLOATS = 4 << 20   # FA_SPLITKV_SCRATCH_FLOATS in include/fa.h

# every symbol include/fa.h declares
EXPORTED = ("fa_fwd", "fa_fwd_validate", "fa_fwd_varlen", "fa_fwd_varlen_validate", "fa_fwd_splitkv",
            "fa_fwd_splitkv_validate", "fa_fwd_splitkv_noalloc", "fa_bwd", "fa_bwd_validate", "fa_bwd_varlen", "fa_bwd_varlen_validate",
            "fa_rotate_quantize_e4m3", "fa_rotate_quantize_validate", "fa_status_string", "fa_version")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load(path: str = LIB_PATH):
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_attention_105_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fp = ctypes.POINTER(ctypes.c_float)
    lib.fa_fwd.restype = i32
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, fp, vp]
    lib.fa_fwd_validate.restype = i32
    lib.fa_fwd_validate.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, fp]
    i64, up = ctypes.c_longlong, ctypes.POINTER(ctypes.c_uint)
    lib.fa_rotate_quantize_e4m3.restype = i32
    lib.fa_rotate_quantize_e4m3.argtypes = [vp, i32, i64, i32, i32, up, vp, vp, vp, vp]
    lib.fa_rotate_quantize_validate.restype = i32
    lib.fa_rotate_quantize_validate.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp]
    lib.fa_fwd_splitkv.restype = i32
    lib.fa_fwd_splitkv.argtypes = [vp] * 5 + [i32] * 7 + [f32, i32, i32, vp, vp]
    lib.fa_fwd_splitkv_validate.restype = i32
    lib.fa_fwd_splitkv_noalloc.restype = i32
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp] * 5 + [i32] * 7 + [f32, i32, i32, vp]
    lib.fa_fwd_splitkv_validate.argtypes = [vp] * 5 + [i32] * 7 + [f32, i32, i32, vp]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_fwd_varlen.argtypes = [vp] * 7 + [i32] * 8 + [f32, i32, vp]
    lib.fa_fwd_varlen_validate.restype = i32
    lib.fa_fwd_varlen_validate.argtypes = [vp] * 7 + [i32] * 8 + [f32, i32]
    lib.fa_bwd.restype = i32
    lib.fa_bwd.argtypes = [vp] * 10 + [i32] * 7 + [f32, i32, vp]
    lib.fa_bwd_validate.restype = i32
    lib.fa_bwd_validate.argtypes = [vp] * 10 + [i32] * 7 + [f32, i32]
    lib.fa_bwd_varlen.restype = i32
    lib.fa_bwd_varlen.argtypes = [vp] * 12 + [i32] * 9 + [f32, i32, vp]
    lib.fa_bwd_varlen_validate.restype = i32
    lib.fa_bwd_varlen_validate.argtypes = [vp] * 12 + [i32] * 9 + [f32, i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i32]
    lib.fa_version.restype = i32
    lib.fa_version.argtypes = []
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _descale_arg(descale):
    if descale is None:
        return None
    arr = (ctypes.c_float * 3)(*[float(x) for x in descale])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)), arr


def fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
           descale, stream) -> int:
    """Raw call of fa_fwd with integer device pointers; returns the status code."""
    ds = _descale_arg(descale)
    return load().fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, int(causal),
                         float(scale), int(dtype), ds[0] if ds else None, stream)


def fa_fwd_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                    dtype, descale) -> int:
    """Raw call of fa_fwd_validate (pure host function); returns the status code."""
    ds = _descale_arg(descale)
    return load().fa_fwd_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d,
                                  int(causal), float(scale), int(dtype), ds[0] if ds else None)


def fa_fwd_splitkv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, n_splits,
                   ws_ptr, stream) -> int:
    """Raw call of fa_fwd_splitkv with integer device pointers; returns the status code."""
    return load().fa_fwd_splitkv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, int(causal),
                                 float(scale), int(dtype), int(n_splits), ws_ptr, stream)


def fa_fwd_splitkv_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
                           n_splits, stream) -> int:
    """Raw call of fa_fwd_splitkv_noalloc (the library's own scratch array
    instead of a workspace); returns the status code."""
    return load().fa_fwd_splitkv_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, int(causal),
                                         float(scale), int(dtype), int(n_splits), stream)


def fa_fwd_splitkv_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype,
                            n_splits, ws_ptr) -> int:
    """Raw call of fa_fwd_splitkv_validate (pure host function)."""
    return load().fa_fwd_splitkv_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Hq, Hkv, Nq, Nk, d,
                                          int(causal), float(scale), int(dtype), int(n_splits), ws_ptr)


def fa_fwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cuq_ptr, cuk_ptr, n_seqs, max_seqlen_q, total_q,
                  total_k, Hq, Hkv, d, causal, scale, dtype, stream) -> int:
    """Raw call of fa_fwd_varlen with integer device pointers; returns the status code."""
    return load().fa_fwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cuq_ptr, cuk_ptr, n_seqs, max_seqlen_q,
                                total_q, total_k, Hq, Hkv, d, int(causal), float(scale), int(dtype), stream)


def fa_fwd_varlen_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cuq_ptr, cuk_ptr, n_seqs, max_seqlen_q,
                           total_q, total_k, Hq, Hkv, d, causal, scale, dtype) -> int:
    """Raw call of fa_fwd_varlen_validate (pure host function)."""
    return load().fa_fwd_varlen_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cuq_ptr, cuk_ptr, n_seqs,
                                         max_seqlen_q, total_q, total_k, Hq, Hkv, d, int(causal),
                                         float(scale), int(dtype))


def fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, B, Hq, Hkv, Nq,
           Nk, d, causal, scale, dtype, stream) -> int:
    """Raw call of fa_bwd with integer device pointers; returns the status code."""
    return load().fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, B, Hq,
                         Hkv, Nq, Nk, d, int(causal), float(scale), int(dtype), stream)


def fa_bwd_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, B, Hq, Hkv,
                    Nq, Nk, d, causal, scale, dtype) -> int:
    """Raw call of fa_bwd_validate (pure host function); returns the status code."""
    return load().fa_bwd_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr,
                                  B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale), int(dtype))


def fa_bwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, cuq_ptr, cuk_ptr,
                  n_seqs, max_seqlen_q, max_seqlen_k, total_q, total_k, Hq, Hkv, d, causal, scale, dtype,
                  stream) -> int:
    """Raw call of fa_bwd_varlen with integer device pointers; returns the status code."""
    return load().fa_bwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr,
                                cuq_ptr, cuk_ptr, n_seqs, max_seqlen_q, max_seqlen_k, total_q, total_k, Hq, Hkv, d,
                                int(causal), float(scale), int(dtype), stream)


def fa_bwd_varlen_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, cuq_ptr,
                           cuk_ptr, n_seqs, max_seqlen_q, max_seqlen_k, total_q, total_k, Hq, Hkv, d, causal,
                           scale, dtype) -> int:
    """Raw call of fa_bwd_varlen_validate (pure host function)."""
    return load().fa_bwd_varlen_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr,
                                         ws_ptr, cuq_ptr, cuk_ptr, n_seqs, max_seqlen_q, max_seqlen_k, total_q,
                                         total_k, Hq, Hkv, d, int(causal), float(scale), int(dtype))


def _sign_bits_arg(sign_bits):
    if sign_bits is None:
        return None, None
    arr = (ctypes.c_uint * len(sign_bits))(*[int(w) for w in sign_bits])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint)), arr


def fa_rotate_quantize_e4m3(x_ptr, x_dtype, rows, d, rotate, sign_bits, codes_ptr, scale_ptr,
                            work_ptr, stream) -> int:
    """Raw call of fa_rotate_quantize_e4m3; ``sign_bits`` is a sequence of
    d/32 words (host) or None.  Returns the status code."""
    bits, keep = _sign_bits_arg(sign_bits)
    return load().fa_rotate_quantize_e4m3(x_ptr, int(x_dtype), int(rows), int(d), int(rotate), bits,
                                          codes_ptr, scale_ptr, work_ptr, stream)


def fa_rotate_quantize_validate(x_ptr, x_dtype, rows, d, rotate, codes_ptr, scale_ptr, work_ptr) -> int:
    """Raw call of fa_rotate_quantize_validate (pure host function)."""
    return load().fa_rotate_quantize_validate(x_ptr, int(x_dtype), int(rows), int(d), int(rotate),
                                              codes_ptr, scale_ptr, work_ptr)


def version() -> int:
    return load().fa_version()
