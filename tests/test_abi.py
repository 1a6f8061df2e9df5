"""The C ABI: the built library exports every function include/fa.h declares,
and fa_fwd_validate (a pure host function) enforces the documented contract.
CPU only: no kernel is launched here."""
import ctypes
import math
import os
import re

import pytest

from exact_attention_105_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_header_declares_the_binding_names():
    assert declared_functions() == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libfa.so does not export {name}"
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert _lib.version() >= 100
    for st in range(4):
        assert _lib.status_string(st).startswith("FA_")
    assert "unknown" in _lib.status_string(99)


GOOD = dict(q=4096, k=8192, v=12288, o=16384, lse=20480, B=2, Hq=8, Hkv=2, Nq=100, Nk=77, d=128,
            causal=1, scale=0.125, dtype=_lib.FA_DTYPE_BF16, descale=None)


def validate(**kw):
    a = dict(GOOD)
    a.update(kw)
    return _lib.fa_fwd_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"],
                                a["descale"])


def test_valid_arguments(lib):
    assert validate() == _lib.FA_SUCCESS
    assert validate(d=64, causal=0) == _lib.FA_SUCCESS
    assert validate(lse=None) == _lib.FA_SUCCESS
    assert validate(scale=0.0) == _lib.FA_SUCCESS
    assert validate(scale=-0.5) == _lib.FA_SUCCESS
    assert validate(B=0, Nk=0, q=None, k=None, v=None, o=None) == _lib.FA_SUCCESS   # nothing to compute
    assert validate(Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None) == _lib.FA_SUCCESS
    assert validate(Nq=0, q=None, o=None, lse=None) == _lib.FA_SUCCESS
    assert validate(B=0, q=None, k=None, v=None, o=None) == _lib.FA_SUCCESS
    assert validate(dtype=_lib.FA_DTYPE_FP8_E4M3, descale=(0.01, 0.02, 0.03)) == _lib.FA_SUCCESS


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(Hq=0), dict(Hkv=0), dict(Nq=-1), dict(Nk=-5), dict(d=0),
    dict(Hq=6, Hkv=4), dict(causal=2), dict(scale=math.inf), dict(scale=math.nan),
    dict(dtype=7), dict(descale=(1.0, 1.0, 1.0)),
    dict(dtype=_lib.FA_DTYPE_FP8_E4M3, descale=None),
    dict(dtype=_lib.FA_DTYPE_FP8_E4M3, descale=(1.0, 0.0, 1.0)),
    dict(dtype=_lib.FA_DTYPE_FP8_E4M3, descale=(1.0, -1.0, 1.0)),
    dict(dtype=_lib.FA_DTYPE_FP8_E4M3, descale=(1.0, 1.0, math.inf)),
    dict(q=None), dict(o=None), dict(k=None), dict(v=None),
    dict(q=4096 + 8), dict(k=8192 + 2), dict(o=16384 + 4), dict(lse=20480 + 2),
    dict(B=1 << 12, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 10, d=128),
    dict(Nk=0, k=None, v=None), dict(Nk=0),                 # rows to compute, no key
])
def test_invalid_arguments(lib, kw):
    assert validate(**kw) == _lib.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(d=32),
                                dict(dtype=_lib.FA_DTYPE_FP8_E4M3, descale=(1.0, 1.0, 1.0), d=64)])
def test_unsupported_combinations(lib, kw):
    assert validate(**kw) == _lib.FA_ERROR_NOT_SUPPORTED


# ---------------------------------------------------------------- fa_rotate_quantize_e4m3
RGOOD = dict(x=4096, x_dtype=_lib.FA_DTYPE_F32, rows=1000, d=128, rotate=1, codes=8192, scale=12288,
             work=12292)


def rvalidate(**kw):
    a = dict(RGOOD)
    a.update(kw)
    return _lib.fa_rotate_quantize_validate(a["x"], a["x_dtype"], a["rows"], a["d"], a["rotate"],
                                            a["codes"], a["scale"], a["work"])


def test_rotate_valid_arguments(lib):
    assert rvalidate() == _lib.FA_SUCCESS
    assert rvalidate(x_dtype=_lib.FA_DTYPE_BF16, d=64, rotate=0) == _lib.FA_SUCCESS
    assert rvalidate(rows=0, x=None, codes=None) == _lib.FA_SUCCESS    # scale still written


@pytest.mark.parametrize("kw", [
    dict(rows=-1), dict(d=0), dict(rotate=2), dict(x_dtype=9), dict(scale=None), dict(work=None),
    dict(x=None), dict(codes=None), dict(x=4096 + 4), dict(x=4096 + 8), dict(codes=8192 + 1),
    dict(codes=8192 + 4), dict(codes=8192 + 8), dict(scale=12288 + 2),
    dict(rows=1 << 24, d=128),
])
def test_rotate_invalid_arguments(lib, kw):
    assert rvalidate(**kw) == _lib.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(d=32), dict(x_dtype=_lib.FA_DTYPE_FP8_E4M3)])
def test_rotate_unsupported(lib, kw):
    assert rvalidate(**kw) == _lib.FA_ERROR_NOT_SUPPORTED


def test_fwd_rejects_fp32_attention(lib):
    assert validate(dtype=_lib.FA_DTYPE_F32) == _lib.FA_ERROR_NOT_SUPPORTED
    assert validate(dtype=_lib.FA_DTYPE_F32, descale=(1.0, 1.0, 1.0)) == _lib.FA_ERROR_INVALID_VALUE


# ---------------------------------------------------------------- fa_bwd
BGOOD = dict(q=4096, k=8192, v=12288, o=16384, lse=20480, do=24576, dq=28672, dk=32768, dv=36864,
             ws=40960, B=2, Hq=8, Hkv=2, Nq=100, Nk=77, d=128, causal=1, scale=0.125,
             dtype=_lib.FA_DTYPE_BF16)


def bvalidate(**kw):
    a = dict(BGOOD)
    a.update(kw)
    return _lib.fa_bwd_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                a["ws"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"],
                                a["scale"], a["dtype"])


def test_bwd_valid_arguments(lib):
    assert bvalidate() == _lib.FA_SUCCESS
    assert bvalidate(d=64, causal=0, Hkv=8) == _lib.FA_SUCCESS
    assert bvalidate(scale=-0.5) == _lib.FA_SUCCESS
    # no query rows: the query-side pointers may be null
    assert bvalidate(Nq=0, q=None, o=None, lse=None, do=None, dq=None, ws=None) == _lib.FA_SUCCESS
    # no query rows and no keys: nothing to compute, every pointer may be null
    assert bvalidate(Nq=0, Nk=0, q=None, o=None, lse=None, do=None, dq=None, ws=None,
                     k=None, v=None, dk=None, dv=None) == _lib.FA_SUCCESS
    assert bvalidate(B=0, Nk=0) == _lib.FA_SUCCESS


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(Hq=0), dict(Hkv=3), dict(Nq=-1), dict(Nk=-2), dict(d=0), dict(causal=2),
    dict(scale=math.inf), dict(scale=math.nan), dict(dtype=7),
    dict(q=None), dict(o=None), dict(lse=None), dict(do=None), dict(dq=None), dict(ws=None),
    dict(k=None), dict(v=None), dict(dk=None), dict(dv=None),
    dict(q=4096 + 8), dict(do=24576 + 2), dict(dq=28672 + 4), dict(dk=32768 + 8), dict(dv=36864 + 1),
    dict(lse=20480 + 2), dict(ws=40960 + 1),
    dict(B=1, Hq=1, Hkv=1, Nq=1 << 24, d=128),
    dict(Nk=0), dict(Nk=0, k=None, v=None, dk=None, dv=None),   # rows to differentiate and no key
])
def test_bwd_invalid_arguments(lib, kw):
    assert bvalidate(**kw) == _lib.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(dtype=_lib.FA_DTYPE_FP8_E4M3),
                                dict(dtype=_lib.FA_DTYPE_F32)])
def test_bwd_unsupported(lib, kw):
    assert bvalidate(**kw) == _lib.FA_ERROR_NOT_SUPPORTED


# ---------------------------------------------------------------- fa_fwd_varlen
VGOOD = dict(q=4096, k=8192, v=12288, o=16384, lse=20480, cuq=24576, cuk=28672, n_seqs=3, max_seqlen_q=700,
             total_q=1000, total_k=1200, Hq=8, Hkv=2, d=128, causal=1, scale=0.125, dtype=_lib.FA_DTYPE_BF16)


def vvalidate(**kw):
    a = dict(VGOOD)
    a.update(kw)
    return _lib.fa_fwd_varlen_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cuq"], a["cuk"], a["n_seqs"],
                                       a["max_seqlen_q"], a["total_q"], a["total_k"], a["Hq"], a["Hkv"], a["d"],
                                       a["causal"], a["scale"], a["dtype"])


def test_varlen_valid_arguments(lib):
    assert vvalidate() == _lib.FA_SUCCESS
    assert vvalidate(d=64, causal=0, lse=None) == _lib.FA_SUCCESS
    assert vvalidate(n_seqs=0, cuq=None, cuk=None) == _lib.FA_SUCCESS
    assert vvalidate(total_k=0, k=None, v=None) == _lib.FA_SUCCESS


@pytest.mark.parametrize("kw", [
    dict(n_seqs=-1), dict(max_seqlen_q=-1), dict(total_q=-1), dict(total_k=-1), dict(Hq=0), dict(Hkv=3),
    dict(d=0), dict(causal=5), dict(scale=math.inf), dict(dtype=9), dict(cuq=None), dict(cuk=None),
    dict(cuq=24576 + 2), dict(q=None), dict(o=None), dict(k=None), dict(v=None), dict(q=4096 + 8),
    dict(o=16384 + 2), dict(lse=20480 + 1), dict(total_q=1 << 22, Hq=8, d=128),
    dict(max_seqlen_q=1 << 30, n_seqs=1 << 10),
])
def test_varlen_invalid_arguments(lib, kw):
    assert vvalidate(**kw) == _lib.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(d=96), dict(dtype=_lib.FA_DTYPE_FP8_E4M3), dict(dtype=_lib.FA_DTYPE_F32)])
def test_varlen_unsupported(lib, kw):
    assert vvalidate(**kw) == _lib.FA_ERROR_NOT_SUPPORTED


# ---------------------------------------------------------------- fa_fwd_splitkv
SGOOD = dict(q=4096, k=8192, v=12288, o=16384, lse=20480, B=1, Hq=32, Hkv=8, Nq=1, Nk=65536, d=128, causal=1,
             scale=0.088, dtype=_lib.FA_DTYPE_BF16, n_splits=16, ws=24576)


def svalidate(**kw):
    a = dict(SGOOD)
    a.update(kw)
    return _lib.fa_fwd_splitkv_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                        a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"],
                                        a["n_splits"], a["ws"])


def test_splitkv_valid_arguments(lib):
    assert svalidate() == _lib.FA_SUCCESS
    assert svalidate(n_splits=1, ws=None) == _lib.FA_SUCCESS
    assert svalidate(Nq=16, n_splits=256) == _lib.FA_SUCCESS
    assert svalidate(B=0, ws=None) == _lib.FA_SUCCESS


@pytest.mark.parametrize("kw", [dict(n_splits=0), dict(n_splits=257), dict(ws=None), dict(ws=24576 + 8),
                                dict(q=None), dict(Hkv=3), dict(dtype=11), dict(scale=math.nan),
                                dict(B=64, Nq=16, n_splits=256)])
def test_splitkv_invalid_arguments(lib, kw):
    assert svalidate(**kw) == _lib.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(d=64), dict(Nq=17), dict(dtype=_lib.FA_DTYPE_FP8_E4M3),
                                dict(dtype=_lib.FA_DTYPE_F32)])
def test_splitkv_unsupported(lib, kw):
    assert svalidate(**kw) == _lib.FA_ERROR_NOT_SUPPORTED


def noalloc(**kw):
    """fa_fwd_splitkv_noalloc on arguments it rejects before any HIP call
    (fake device pointers, null stream): nothing is launched."""
    a = dict(SGOOD)
    a.update(kw)
    return _lib.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                       a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"], a["n_splits"], None)


@pytest.mark.parametrize("kw", [dict(n_splits=0), dict(q=None), dict(Hkv=3), dict(scale=math.nan),
                                dict(B=64, Nq=16, n_splits=256),
                                dict(B=32, Nq=2, n_splits=16)])     # 16*32*32*2*129 floats > 4 Mi
def test_splitkv_noalloc_invalid_arguments(lib, kw):
    assert noalloc(**kw) == _lib.FA_ERROR_INVALID_VALUE


def test_splitkv_noalloc_scratch_limit_is_the_header_constant():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_SPLITKV_SCRATCH_FLOATS \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.SPLITKV_SCRATCH_FLOATS
    # largest accepted problem at 16 splits, d = 128: 16 * 2032 rows * 129 floats
    assert 16 * 2032 * 129 <= _lib.SPLITKV_SCRATCH_FLOATS < 16 * 2033 * 129


@pytest.mark.parametrize("kw", [dict(d=64), dict(Nq=17), dict(dtype=_lib.FA_DTYPE_FP8_E4M3)])
def test_splitkv_noalloc_unsupported(lib, kw):
    assert noalloc(**kw) == _lib.FA_ERROR_NOT_SUPPORTED


# ---------------------------------------------------------------- fa_bwd_varlen
BVGOOD = dict(q=4096, k=8192, v=12288, o=16384, lse=20480, do=24576, dq=28672, dk=32768, dv=36864, ws=40960,
              cuq=45056, cuk=49152, n_seqs=3, max_q=700, max_k=800, total_q=1000, total_k=1200, Hq=8, Hkv=2,
              d=128, causal=1, scale=0.125, dtype=_lib.FA_DTYPE_BF16)


def bvvalidate(**kw):
    a = dict(BVGOOD)
    a.update(kw)
    return _lib.fa_bwd_varlen_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                       a["ws"], a["cuq"], a["cuk"], a["n_seqs"], a["max_q"], a["max_k"],
                                       a["total_q"], a["total_k"], a["Hq"], a["Hkv"], a["d"], a["causal"],
                                       a["scale"], a["dtype"])


def test_bwd_varlen_valid_arguments(lib):
    assert bvvalidate() == _lib.FA_SUCCESS
    assert bvvalidate(d=64, causal=0) == _lib.FA_SUCCESS
    assert bvvalidate(n_seqs=0, cuq=None, cuk=None) == _lib.FA_SUCCESS


@pytest.mark.parametrize("kw", [dict(n_seqs=-1), dict(max_k=-1), dict(total_q=-1), dict(Hkv=3), dict(cuk=None),
                                dict(ws=None), dict(dq=None), dict(dk=None), dict(dv=28672 + 8),
                                dict(lse=20480 + 2), dict(scale=math.inf), dict(dtype=5),
                                dict(total_k=1 << 22, Hkv=8, d=128)])
def test_bwd_varlen_invalid_arguments(lib, kw):
    assert bvvalidate(**kw) == _lib.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(d=96), dict(dtype=_lib.FA_DTYPE_FP8_E4M3)])
def test_bwd_varlen_unsupported(lib, kw):
    assert bvvalidate(**kw) == _lib.FA_ERROR_NOT_SUPPORTED
