"""Python face of the exact-attention oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and
its binding) never imports it.

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double, OpenMP over
query rows).  This wrapper only marshals numpy arrays into that library:

* ``attention``   -- O and LSE by the naive definition (page "FlashAttention
  (DE)", systems-analysis.info, section "Problematik der Standard-Attention")
  or by the online-softmax recurrence (same page, section
  "Online-Softmax-Berechnung") when ``block_keys > 0``;
* ``probs_row``   -- one materialised row of P;
* ``decode``      -- the oracle's own bfloat16 / OCP-E4M3 decoders;
* ``rotate``, ``quantize_e4m3``, ``e4m3_encode`` -- the random-sign Hadamard
  rotation and per-tensor FP8 quantisation of page "FlashAttention-3 (DE)",
  systems-analysis.ru, technical innovation 3 (``rotate_oracle.c``);
* ``attention_bwd``, ``bwd_dq_rows`` -- the gradients dQ, dK, dV of
  attention by the chain rule through the definition (``attn_bwd_oracle.c``).

Inputs are the exact bytes the GPU receives: ``uint16`` arrays holding
bfloat16 bit patterns, ``uint8`` arrays holding E4M3 codes (plus per-tensor
scales), or ``float64`` arrays for hand-made cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_ROT_SRC = os.path.join(_HERE, "rotate_oracle.c")
_BWD_SRC = os.path.join(_HERE, "attn_bwd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"bf16": 0, "e4m3": 1, "f64": 2}
_NP = {"bf16": np.uint16, "e4m3": np.uint8, "f64": np.float64}

_default = None


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH, rot_src: str = _ROT_SRC,
          bwd_src: str = _BWD_SRC, sanitize: bool = False) -> str:
    """Compile the oracle C sources into a shared library with gcc (IEEE semantics);
    ``sanitize`` adds AddressSanitizer and UndefinedBehaviorSanitizer (a test
    build: load it in a process that preloads libasan)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", *(SANITIZE_FLAGS if sanitize else []),
               src, rot_src, bwd_src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


class OracleLib:
    """One loaded copy of the oracle library (the default one, or a test's mutant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [vp, vp, vp, ctypes.c_int, dp, i64, i64, i64, i64, i64,
                                         i64, ctypes.c_int, ctypes.c_double, ctypes.POINTER(i64),
                                         i64, i64, dp, dp]
        lib.oracle_probs_row.restype = ctypes.c_int
        lib.oracle_probs_row.argtypes = [vp, vp, vp, ctypes.c_int, dp, i64, i64, i64, i64, i64,
                                         i64, ctypes.c_int, ctypes.c_double, i64, dp]
        lib.oracle_decode.restype = None
        lib.oracle_decode.argtypes = [vp, ctypes.c_int, ctypes.c_double, i64, dp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_rotate.restype = ctypes.c_int
        lib.oracle_rotate.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.POINTER(ctypes.c_uint32),
                                      ctypes.c_int, dp]
        lib.oracle_quantize_e4m3.restype = None
        lib.oracle_quantize_e4m3.argtypes = [dp, i64, dp, ctypes.POINTER(ctypes.c_uint8)]
        lib.oracle_encode_scaled.restype = None
        lib.oracle_encode_scaled.argtypes = [dp, i64, ctypes.c_double, ctypes.POINTER(ctypes.c_uint8)]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_hadamard_entry.restype = ctypes.c_double
        lib.oracle_hadamard_entry.argtypes = [i64, i64]
        lib.oracle_attention_bwd.restype = ctypes.c_int
        lib.oracle_attention_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                             ctypes.c_int, ctypes.c_double, dp, dp, dp]
        lib.oracle_bwd_dq_rows.restype = ctypes.c_int
        lib.oracle_bwd_dq_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                           ctypes.c_int, ctypes.c_double, ctypes.POINTER(i64), i64, dp]
        self.lib = lib
        self.path = path

    def attention(self, q, k, v, *, causal, scale, dtype="bf16", descale=None, rows=None,
                  block_keys=0):
        return _attention(self.lib, q, k, v, causal, scale, dtype, descale, rows, block_keys)

    def probs_row(self, q, k, v, *, causal, scale, row, dtype="bf16", descale=None):
        return _probs_row(self.lib, q, k, v, causal, scale, row, dtype, descale)

    def decode(self, codes, dtype, descale=1.0):
        return _decode(self.lib, codes, dtype, descale)

    def attention_bwd(self, q, k, v, dout, *, causal, scale, dtype="bf16"):
        return _attention_bwd(self.lib, q, k, v, dout, causal, scale, dtype)

    def bwd_dq_rows(self, q, k, v, dout, *, causal, scale, rows, dtype="bf16"):
        return _bwd_dq_rows(self.lib, q, k, v, dout, causal, scale, rows, dtype)

    def num_threads(self):
        return int(self.lib.oracle_num_threads())

    def rotate(self, x, *, signs=None, rotate=True):
        return _rotate(self.lib, x, signs, rotate)

    def quantize_e4m3(self, y):
        return _quantize(self.lib, y)

    def encode_scaled(self, y, s):
        y = np.ascontiguousarray(y, dtype=np.float64)
        codes = np.empty(y.shape, dtype=np.uint8)
        self.lib.oracle_encode_scaled(_dptr(y), y.size, float(s),
                                      codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
        return codes

    def e4m3_encode(self, v):
        return int(self.lib.oracle_e4m3_encode(float(v)))

    def hadamard_entry(self, i, j):
        return float(self.lib.oracle_hadamard_entry(int(i), int(j)))


def default() -> OracleLib:
    """The oracle built from its C sources (rebuilt when a source is newer)."""
    global _default
    if _default is None:
        newest = max(os.path.getmtime(_SRC), os.path.getmtime(_ROT_SRC), os.path.getmtime(_BWD_SRC))
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
            build(force=True)
        _default = OracleLib(_LIB_PATH)
    return _default


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(q, k, v, dtype):
    want = _NP[dtype]
    arrs = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        t = np.ascontiguousarray(t)
        if t.dtype != want:
            raise TypeError(f"{name}: expected {np.dtype(want)} for dtype {dtype}, got {t.dtype}")
        if t.ndim != 4:
            raise ValueError(f"{name}: expected [B, H, N, d], got shape {t.shape}")
        arrs.append(t)
    q, k, v = arrs
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return q, k, v, (B, Hq, Hkv, Nq, Nk, d)


def _descale(dtype, descale):
    if dtype != "e4m3":
        return None
    if descale is None or len(descale) != 3:
        raise ValueError("e4m3 inputs need descale = (dq, dk, dv)")
    return np.ascontiguousarray(np.asarray(descale, dtype=np.float64))


def _attention(lib, q, k, v, causal, scale, dtype, descale, rows, block_keys):
    """Return (O, LSE) in float64.

    Without ``rows`` the shapes are O [B,Hq,Nq,d] and LSE [B,Hq,Nq]; with
    ``rows`` (flat indices (b*Hq + h)*Nq + i) they are [n,d] and [n].
    """
    q, k, v, (B, Hq, Hkv, Nq, Nk, d) = _prep(q, k, v, dtype)
    ds = _descale(dtype, descale)
    if rows is None:
        n = B * Hq * Nq
        rows_arr, rows_ptr = None, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
        rows_ptr = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    o = np.zeros((max(n, 1), d), dtype=np.float64)
    lse = np.zeros(max(n, 1), dtype=np.float64)
    rc = lib.oracle_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPES[dtype],
                              _dptr(ds) if ds is not None else None,
                              B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                              rows_ptr, n, int(block_keys), _dptr(o), _dptr(lse))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    o, lse = o[:n], lse[:n]
    if rows is None:
        return o.reshape(B, Hq, Nq, d), lse.reshape(B, Hq, Nq)
    return o, lse


def _probs_row(lib, q, k, v, causal, scale, row, dtype, descale):
    q, k, v, (B, Hq, Hkv, Nq, Nk, d) = _prep(q, k, v, dtype)
    ds = _descale(dtype, descale)
    p = np.zeros(max(Nk, 1), dtype=np.float64)
    rc = lib.oracle_probs_row(q.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPES[dtype],
                              _dptr(ds) if ds is not None else None,
                              B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                              int(row), _dptr(p))
    if rc < 0:
        raise ValueError("oracle_probs_row rejected its arguments")
    return p[:Nk]


def _prep_bwd(q, k, v, dout, dtype):
    if dtype not in ("bf16", "f64"):
        raise ValueError("the backward oracle takes bf16 or f64 inputs")
    q, k, v, dims = _prep(q, k, v, dtype)
    dout = np.ascontiguousarray(dout)
    if dout.dtype != q.dtype or dout.shape != q.shape:
        raise ValueError(f"dout must match q: {dout.dtype}{dout.shape} vs {q.dtype}{q.shape}")
    return q, k, v, dout, dims


def _attention_bwd(lib, q, k, v, dout, causal, scale, dtype):
    """Return (dQ, dK, dV) in float64, shaped like q, k, v."""
    q, k, v, dout, (B, Hq, Hkv, Nq, Nk, d) = _prep_bwd(q, k, v, dout, dtype)
    dq = np.zeros((B, Hq, Nq, d), dtype=np.float64)
    dk = np.zeros((B, Hkv, Nk, d), dtype=np.float64)
    dv = np.zeros((B, Hkv, Nk, d), dtype=np.float64)
    rc = lib.oracle_attention_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                  DTYPES[dtype], B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                  _dptr(dq), _dptr(dk), _dptr(dv))
    if rc != 0:
        raise ValueError("oracle_attention_bwd rejected its arguments")
    return dq, dk, dv


def _bwd_dq_rows(lib, q, k, v, dout, causal, scale, rows, dtype):
    """dQ of the listed rows (flat (b*Hq + h)*Nq + i), [n, d] float64."""
    q, k, v, dout, (B, Hq, Hkv, Nq, Nk, d) = _prep_bwd(q, k, v, dout, dtype)
    rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((max(rows_arr.size, 1), d), dtype=np.float64)
    rc = lib.oracle_bwd_dq_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                DTYPES[dtype], B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows_arr.size,
                                _dptr(out))
    if rc != 0:
        raise ValueError("oracle_bwd_dq_rows rejected its arguments")
    return out[:rows_arr.size]


def _decode(lib, codes, dtype, descale):
    codes = np.ascontiguousarray(codes)
    if codes.dtype != _NP[dtype]:
        raise TypeError(f"expected {np.dtype(_NP[dtype])} codes for {dtype}")
    out = np.empty(codes.size, dtype=np.float64)
    lib.oracle_decode(codes.ctypes.data, DTYPES[dtype], float(descale), codes.size, _dptr(out))
    return out.reshape(codes.shape)


def attention(q, k, v, *, causal: bool, scale: float, dtype: str = "bf16", descale=None,
              rows=None, block_keys: int = 0):
    """Return (O, LSE) in float64.

    Without ``rows`` the shapes are O [B,Hq,Nq,d] and LSE [B,Hq,Nq]; with
    ``rows`` (flat indices (b*Hq + h)*Nq + i) they are [n,d] and [n].
    ``block_keys == 0`` is the naive definition; ``> 0`` the online-softmax
    recurrence over blocks of that many keys.
    """
    return default().attention(q, k, v, causal=causal, scale=scale, dtype=dtype,
                               descale=descale, rows=rows, block_keys=block_keys)


def probs_row(q, k, v, *, causal: bool, scale: float, row: int, dtype: str = "bf16",
              descale=None):
    """The materialised probability row P[row, :] (length Nk) in float64."""
    return default().probs_row(q, k, v, causal=causal, scale=scale, row=row, dtype=dtype,
                               descale=descale)


def decode(codes: np.ndarray, dtype: str, descale: float = 1.0) -> np.ndarray:
    """Decode bfloat16 bit patterns or E4M3 codes to float64 with the oracle's decoders."""
    return default().decode(codes, dtype, descale)


def num_threads() -> int:
    """OpenMP threads the oracle will use (OMP_NUM_THREADS, else all cores)."""
    return default().num_threads()


_ROT_DTYPES = {np.dtype(np.uint16): 0, np.dtype(np.float64): 2, np.dtype(np.float32): 3}


def sign_bits(signs) -> np.ndarray:
    """Pack a length-d sequence of +-1 into the uint32 bit mask the rotation
    takes (bit i set = feature i is negated)."""
    s = np.asarray(signs)
    d = s.size
    words = np.zeros((d + 31) // 32, dtype=np.uint32)
    for i in np.nonzero(s < 0)[0]:
        words[i >> 5] |= np.uint32(1) << np.uint32(i & 31)
    return words


def _rotate(lib, x, signs, rotate):
    """y = x D H / sqrt(d) row by row (x: [..., d] as uint16 bfloat16 bits,
    float32 or float64), in float64; ``signs`` is a length-d +-1 sequence."""
    x = np.ascontiguousarray(x)
    if x.dtype not in _ROT_DTYPES:
        raise TypeError(f"rotate: unsupported dtype {x.dtype}")
    d = x.shape[-1]
    rows = x.size // d if d else 0
    y = np.empty(x.shape, dtype=np.float64)
    bits = None
    if signs is not None:
        bits = np.ascontiguousarray(sign_bits(signs))
        if len(signs) != d:
            raise ValueError("signs must have one entry per feature")
    rc = lib.oracle_rotate(x.ctypes.data, _ROT_DTYPES[x.dtype], rows, d,
                           bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)) if bits is not None else None,
                           int(bool(rotate)), _dptr(y))
    if rc != 0:
        raise ValueError("oracle_rotate rejected its arguments (d must be a power of two)")
    return y


def _quantize(lib, y):
    """Per-tensor E4M3 quantisation: (codes uint8 like y, scale s = amax / 448)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    codes = np.empty(y.shape, dtype=np.uint8)
    s = ctypes.c_double()
    lib.oracle_quantize_e4m3(_dptr(y), y.size, ctypes.byref(s),
                             codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return codes, s.value


def rotate(x, *, signs=None, rotate: bool = True) -> np.ndarray:
    """Rotate every row of x by M = D H / sqrt(d) in float64 (identity when rotate=False)."""
    return default().rotate(x, signs=signs, rotate=rotate)


def quantize_e4m3(y) -> tuple:
    """Per-tensor OCP E4M3 quantisation of float64 values: (codes, scale)."""
    return default().quantize_e4m3(y)


def e4m3_encode(v: float) -> int:
    """The oracle's E4M3 encoder (nearest, ties to even, saturating at 448)."""
    return default().e4m3_encode(v)


def hadamard_entry(i: int, j: int) -> float:
    """Sylvester-Hadamard entry H[i][j] = (-1)^popcount(i & j)."""
    return default().hadamard_entry(i, j)


def encode_scaled(y, s: float) -> np.ndarray:
    """E4M3 codes of y / s (the encoding step of the per-tensor quantisation)."""
    return default().encode_scaled(y, s)


def attention_bwd(q, k, v, dout, *, causal: bool, scale: float, dtype: str = "bf16"):
    """Gradients (dQ, dK, dV) of attention for upstream gradient dout, float64."""
    return default().attention_bwd(q, k, v, dout, causal=causal, scale=scale, dtype=dtype)


def bwd_dq_rows(q, k, v, dout, *, causal: bool, scale: float, rows, dtype: str = "bf16"):
    """dQ of the listed rows (flat (b*Hq + h)*Nq + i) only, [n, d] float64."""
    return default().bwd_dq_rows(q, k, v, dout, causal=causal, scale=scale, rows=rows, dtype=dtype)


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool, scale: float,
                     dtype: str = "bf16"):
    """Attention over a packed batch of variable-length sequences, float64.

    q [total_q, Hq, d], k and v [total_k, Hkv, d] (token-major); sequence s
    owns query tokens cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and key tokens
    cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1 and is an independent attention
    problem.  Returns O [total_q, Hq, d] and LSE [Hq, total_q]; each
    sequence goes through ``attention`` in the [1, H, N, d] layout.
    """
    q, k, v = (np.ascontiguousarray(t) for t in (q, k, v))
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or len(cq) < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold n_seqs + 1 offsets")
    total_q, Hq, d = q.shape
    o = np.zeros((total_q, Hq, d), dtype=np.float64)
    lse = np.full((Hq, total_q), -np.inf, dtype=np.float64)
    for s in range(len(cq) - 1):
        qa, qe, ka, ke = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if qe <= qa:
            continue
        qs = np.ascontiguousarray(q[qa:qe].transpose(1, 0, 2)[None])
        ks = np.ascontiguousarray(k[ka:ke].transpose(1, 0, 2)[None])
        vs = np.ascontiguousarray(v[ka:ke].transpose(1, 0, 2)[None])
        os_, ls = attention(qs, ks, vs, causal=causal, scale=scale, dtype=dtype)
        o[qa:qe] = os_[0].transpose(1, 0, 2)
        lse[:, qa:qe] = ls[0]
    return o, lse


def attention_bwd_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, *, causal: bool, scale: float,
                         dtype: str = "bf16"):
    """Gradients (dQ, dK, dV) of a packed variable-length batch, float64, in
    the packed layouts ([total_q, Hq, d], [total_k, Hkv, d]); each sequence
    goes through ``attention_bwd`` in the [1, H, N, d] layout."""
    q, k, v, dout = (np.ascontiguousarray(t) for t in (q, k, v, dout))
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or len(cq) < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold n_seqs + 1 offsets")
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    to_b = lambda t, a, e: np.ascontiguousarray(t[a:e].transpose(1, 0, 2)[None])
    for s in range(len(cq) - 1):
        qa, qe, ka, ke = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if qe <= qa or ke <= ka:
            continue                      # no query or no key: every gradient of the sequence is 0
        gq, gk, gv = attention_bwd(to_b(q, qa, qe), to_b(k, ka, ke), to_b(v, ka, ke), to_b(dout, qa, qe),
                                   causal=causal, scale=scale, dtype=dtype)
        dq[qa:qe] = gq[0].transpose(1, 0, 2)
        dk[ka:ke] = gk[0].transpose(1, 0, 2)
        dv[ka:ke] = gv[0].transpose(1, 0, 2)
    return dq, dk, dv

