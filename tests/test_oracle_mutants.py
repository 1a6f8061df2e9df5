"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of the oracle's C source with one plausible mistake --
a dropped term, a wrong sign, a wrong index, a swapped operand, a wrong
constant -- compiled into a temporary library.  The pins of
``oracle_pins.py`` are run against it, and at least one must fail.  This is
evidence that the pins constrain every part of the oracle, not a check of
the oracle itself.
"""
import os

import pytest

import oracle
from oracle.oracle import _SRC, OracleLib, build
from oracle_pins import PINS

MUTANTS = {
    "max_not_subtracted_in_lse": ("s[j] = exp(s[j] - M); L += s[j];", "s[j] = exp(s[j]); L += s[j];"),
    "wrong_sign_in_exp": ("s[j] = exp(s[j] - M); L += s[j];", "s[j] = exp(M - s[j]); L += s[j];"),
    "scale_dropped": ("s[j] = p->scale * dot;", "s[j] = dot;"),
    "causal_off_by_one": ("return !p->causal || j <= i + (p->Nk - p->Nq);",
                          "return !p->causal || j < i + (p->Nk - p->Nq);"),
    "causal_top_left": ("return !p->causal || j <= i + (p->Nk - p->Nq);",
                        "return !p->causal || j <= i;"),
    "causal_transposed": ("return !p->causal || j <= i + (p->Nk - p->Nq);",
                          "return !p->causal || j >= i + (p->Nk - p->Nq);"),
    "gqa_interleaved": ("int64_t kvh = h / (p->Hq / p->Hkv);\n    int64_t qoff",
                        "int64_t kvh = h % p->Hkv;\n    int64_t qoff"),
    "lse_without_log": ("*lse = M + log(L);", "*lse = M + L;"),
    "not_normalised": ("for (int64_t j = 0; j < p->Nk; ++j) s[j] /= L;                          /* s now holds P_j */",
                       ""),
    "v_replaced_by_k": ("o[t] += s[j] * load_elem(p->v,", "o[t] += s[j] * load_elem(p->k,"),
    "v_row_index_wrong": ("int64_t voff = ((b * p->Hkv + kvh) * p->Nk + j) * p->d;\n        for (int64_t t = 0; t < p->d; ++t) o[t] += s[j]",
                          "int64_t voff = ((b * p->Hkv + kvh) * p->Nk + (p->Nk - 1 - j)) * p->d;\n        for (int64_t t = 0; t < p->d; ++t) o[t] += s[j]"),
    "q_k_dims_transposed": ("dot += qrow[t] * load_elem(p->k, p->dtype, koff + t, p->dk);",
                            "dot += qrow[t] * load_elem(p->k, p->dtype, koff + (p->d - 1 - t), p->dk);"),
    "empty_row_lse_zero": ("        *lse = -INFINITY;\n        return;\n    }\n    double L = 0.0;",
                           "        *lse = 0.0;\n        return;\n    }\n    double L = 0.0;"),
    "bf16_shift_wrong": ("uint32_t bits = ((uint32_t)h) << 16;", "uint32_t bits = ((uint32_t)h) << 15;"),
    "e4m3_bias_wrong": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal_wrong": ("mag = ldexp((double)m / 8.0, 1 - 7);", "mag = ldexp((double)m / 8.0, -7);"),
    "descale_dropped": ("return oracle_e4m3_to_f64(((const uint8_t*)base)[idx]) * descale;",
                        "return oracle_e4m3_to_f64(((const uint8_t*)base)[idx]);"),
    "descale_q_k_swapped": ("p.dq = descale[0]; p.dk = descale[1]; p.dv = descale[2];\n    }\n    int64_t total",
                            "p.dq = descale[0]; p.dk = descale[2]; p.dv = descale[1];\n    }\n    int64_t total"),
    "tiled_alpha_not_applied_to_l": ("        l *= alpha;\n", ""),
    "tiled_alpha_not_applied_to_o": ("        for (int64_t t = 0; t < p->d; ++t) o[t] *= alpha;\n", ""),
    "tiled_last_block_dropped": ("int64_t j1 = j0 + Bc < p->Nk ? j0 + Bc : p->Nk;",
                                 "int64_t j1 = j0 + Bc < p->Nk ? j0 + Bc : j0;"),
    "probs_not_normalised": ("for (int64_t j = 0; j < Nk; ++j) prow[j] /= L;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = build(force=True, src=str(path), out=str(tmp_path / f"libmut_{name}.so"))
    mut = OracleLib(lib_path)
    failures = []
    for pin in PINS:
        try:
            pin(mut)
        except AssertionError as e:   # the pin caught the planted mistake
            failures.append(pin.__name__)
        except (ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"mutant {name} passed every pin"


def test_unmutated_source_passes_every_pin():
    orc = oracle.default()
    for pin in PINS:
        pin(orc)


# ---------------------------------------------------------------- rotation oracle
from oracle.oracle import _ROT_SRC  # noqa: E402
from rotate_pins import RPINS  # noqa: E402

ROT_MUTANTS = {
    "hadamard_sign_inverted": ("return (popcount64((uint64_t)(i & j)) & 1) ? -1.0 : 1.0;",
                               "return (popcount64((uint64_t)(i & j)) & 1) ? 1.0 : -1.0;"),
    "hadamard_or_instead_of_and": ("return (popcount64((uint64_t)(i & j)) & 1) ? -1.0 : 1.0;",
                                   "return (popcount64((uint64_t)(i | j)) & 1) ? -1.0 : 1.0;"),
    "normalisation_dropped": ("out[j] = acc * norm;", "out[j] = acc;"),
    "signs_ignored": ("if (sign_bits && ((sign_bits[i >> 5] >> (i & 31)) & 1)) xi = -xi;", ""),
    "transposed_product": ("acc += xi * oracle_hadamard_entry(i, j);",
                           "acc += ro_load(x, dtype, r * d + j) * oracle_hadamard_entry(i, j);"),
    "ties_to_odd": ("else c = (lo & 1) ? hi : lo;   /* tie: the even code */",
                    "else c = (lo & 1) ? lo : hi;"),
    "ties_round_up": ("else c = (lo & 1) ? hi : lo;   /* tie: the even code */", "else c = hi;"),
    "no_saturation": ("if (a >= 448.0) return sign | 126;", "if (a >= 480.0) return sign | 127;"),
    "subnormal_scale_wrong": ("return e == 0 ? ldexp((double)m / 8.0, -6)", "return e == 0 ? ldexp((double)m / 8.0, -7)"),
    "scale_uses_240": ("const double s = amax > 0.0 ? amax / 448.0 : 1.0;",
                       "const double s = amax > 0.0 ? amax / 240.0 : 1.0;"),
    "amax_not_absolute": ("double a = fabs(y[k]);", "double a = y[k];"),
}


@pytest.mark.parametrize("name", sorted(ROT_MUTANTS))
def test_rotation_mutant_is_caught(name, tmp_path):
    old, new = ROT_MUTANTS[name]
    src = open(_ROT_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"rmut_{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = build(force=True, rot_src=str(path), out=str(tmp_path / f"librmut_{name}.so"))
    mut = OracleLib(lib_path)
    failures = []
    for pin in RPINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"rotation mutant {name} passed every pin"


def test_unmutated_rotation_source_passes_every_pin():
    orc = oracle.default()
    for pin in RPINS:
        pin(orc)


# ---------------------------------------------------------------- backward oracle
from oracle.oracle import _BWD_SRC  # noqa: E402
from bwd_pins import BPINS  # noqa: E402

BWD_MUTANTS = {
    "jacobian_row_term_dropped": ("r->dprow[j] = r->prow[j] * (r->dprow[j] - Dsum);",
                                  "r->dprow[j] = r->prow[j] * r->dprow[j];"),
    "jacobian_sign_flipped": ("r->dprow[j] = r->prow[j] * (r->dprow[j] - Dsum);",
                              "r->dprow[j] = r->prow[j] * (Dsum - r->dprow[j]);"),
    "row_term_unweighted": ("Dsum += r->prow[j] * r->dprow[j];", "Dsum += r->dprow[j];"),
    "dq_scale_dropped": ("dqi[t] += scale * ds * bw_load(k, dtype, koff + t);",
                         "dqi[t] += ds * bw_load(k, dtype, koff + t);"),
    "dk_scale_squared": ("dk[koff + t] += scale * ds * r.qrow[t];",
                         "dk[koff + t] += scale * scale * ds * r.qrow[t];"),
    "dk_uses_do": ("dk[koff + t] += scale * ds * r.qrow[t];", "dk[koff + t] += scale * ds * r.dorow[t];"),
    "dv_uses_ds": ("dv[koff + t] += pj * r.dorow[t];", "dv[koff + t] += ds * r.dorow[t];"),
    "dv_uses_q": ("dv[koff + t] += pj * r.dorow[t];", "dv[koff + t] += pj * r.qrow[t];"),
    "dp_uses_k": ("for (int64_t t = 0; t < d; ++t) dot += r->dorow[t] * bw_load(p->v, p->dtype, voff + t);",
                  "for (int64_t t = 0; t < d; ++t) dot += r->dorow[t] * bw_load(p->k, p->dtype, voff + t);"),
    "softmax_not_normalised": ("for (int64_t j = 0; j < Nk; ++j) r->prow[j] /= L;", ""),
    "causal_off_by_one": ("if (p->causal && j > i + (Nk - p->Nq))", "if (p->causal && j >= i + (Nk - p->Nq))"),
    "causal_top_left": ("if (p->causal && j > i + (Nk - p->Nq))", "if (p->causal && j > i)"),
    "gqa_interleaved": ("    const int64_t kvh = h / (p->Hq / p->Hkv);", "    const int64_t kvh = h % p->Hkv;"),
    "key_row_reversed": ("const int64_t koff = ((b * Hkv + kvh) * Nk + j) * d;\n                            for",
                         "const int64_t koff = ((b * Hkv + kvh) * Nk + (Nk - 1 - j)) * d;\n                            for"),
    "scale_missing_in_scores": ("r->prow[j] = p->scale * dot;", "r->prow[j] = dot;"),
    "rows_dq_uses_v": ("out[t] += scale * r.dprow[j] * bw_load(k, dtype, koff + t);",
                       "out[t] += scale * r.dprow[j] * bw_load(v, dtype, koff + t);"),
    "bf16_shift_wrong": ("uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;",
                         "uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 15;"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = open(_BWD_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"bmut_{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = build(force=True, bwd_src=str(path), out=str(tmp_path / f"libbmut_{name}.so"))
    mut = OracleLib(lib_path)
    failures = []
    for pin in BPINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"backward mutant {name} passed every pin"


def test_unmutated_backward_source_passes_every_pin():
    orc = oracle.default()
    for pin in BPINS:
        pin(orc)

