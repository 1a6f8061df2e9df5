"""Exact-attention oracle -- TEST INFRASTRUCTURE, not part of the product.

A plain fp64 CPU implementation of softmax(scale * Q K^T + mask) V and its
per-row log-sum-exp.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the HIP library and its
Python binding never do, and nothing here is shared with them.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
and ``tests/test_codecs.py`` (closed-form hand cases, invariants, brute force,
library cross-checks).  The GPU-versus-oracle tolerances themselves come
from the project's stated acceptance bounds, not from the pages.
"""
from .oracle import (OracleLib, attention, build, decode, default, num_threads,  # noqa: F401
                     probs_row)
