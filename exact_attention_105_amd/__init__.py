"""Fused exact-attention forward pass for AMD MI355X (gfx950), HIP kernels behind a C ABI.

``fwd(q, k, v, causal=..., scale=..., descale=...) -> (O, LSE)`` computes
softmax(scale * Q K^T + mask) V and the per-row log-sum-exp in one kernel
that never writes the score matrix to device memory.
``bwd(q, k, v, o, lse, dout, ...) -> (dQ, dK, dV)`` is its backward pass,
recomputing the probabilities from LSE; ``fwd_varlen`` runs a packed batch of
sequences of different lengths; ``fwd_splitkv`` splits the keys of decode
shapes over several workgroups when few (batch, head) units exist.
``rotate_quantize(x, signs=...) -> (codes, scale)`` is the random-sign
Hadamard rotation and per-tensor E4M3 quantisation that prepares Q and K for
the FP8 kernel.  The C ABI is declared in include/fa.h; ``_lib`` is its
ctypes binding.
"""
from ._lib import EXPORTED, FaError, load, status_string, version  # noqa: F401
from .attention import (bwd, bwd_varlen, default_splits, fwd, fwd_splitkv, fwd_splitkv_noalloc,  # noqa: F401
                        fwd_varlen, rotate_quantize, sign_bits)
