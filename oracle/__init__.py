"""Exact-attention oracle -- TEST INFRASTRUCTURE, not part of the product.

A plain fp64 CPU implementation of softmax(scale * Q K^T + mask) V and its
per-row log-sum-exp, of its gradients dQ, dK, dV, and of the random-sign
Hadamard rotation with per-tensor FP8 (E4M3) quantisation that precedes
low-precision attention.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the HIP library and its
Python binding never do, and nothing here is shared with them.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_rotate_pins.py``, ``tests/test_bwd_pins.py`` and
``tests/test_codecs.py`` (closed-form hand cases, invariants, brute force,
finite differences, library cross-checks).  The GPU-versus-oracle tolerances
themselves come from the project's stated acceptance bounds (forward) and
from the arithmetic of the kernels (backward, rotation), not from the pages.
"""
from .oracle import (OracleLib, attention, attention_bwd, attention_bwd_varlen, attention_varlen,  # noqa: F401
                     build, bwd_dq_rows, decode, default, e4m3_encode, encode_scaled, hadamard_entry,
                     num_threads, probs_row, quantize_e4m3, rotate, sign_bits)
