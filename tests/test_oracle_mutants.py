"""CPU test: the pins are strong enough to catch plausible oracle mistakes.

Each mutant is a copy of oracle/mla_oracle.c with one deliberate error (a
dropped term, a wrong sign or index, a transposed operand, a wrong slice),
compiled with gcc into a temporary directory.  The real oracle passes every
pin; each mutant must fail at least one.
"""
import os
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.c")

MUTANTS = {
    "drop_rotary_term": ("s[j] = (lat + rot) * scale;", "s[j] = (lat) * scale;"),
    "drop_scale": ("s[j] = (lat + rot) * scale;", "s[j] = (lat + rot);"),
    "transpose_w_uk": ("qn[d] * w_uk[d * Dc + c]", "qn[d] * w_uk[c * Dn + d]"),
    "transpose_w_uv": ("mix[c] * w_uv[d * Dc + c]", "mix[c] * w_uv[c * Dv + d]"),
    "w_uv_from_w_uk_rows": ("(h * rows_per_head + Dn) * Dc", "(h * rows_per_head) * Dc"),
    "softmax_sign": ("denom += exp(s[j] - m)", "denom += exp(m - s[j])"),
    "mix_wrong_row": ("const double* crow = kv + b * kv_sb + set[j] * kv_st;\n                for (int64_t c = 0; c < Dc; ++c) mix",
                      "const double* crow = kv + b * kv_sb + set[0] * kv_st;\n                for (int64_t c = 0; c < Dc; ++c) mix"),
    "mask_off_by_one": ("mark[t] = 1;", "mark[t > 0 ? t - 1 : t] = 1;"),
    "rotary_uses_latent": ("const double* prow = pe + b * pe_sb + set[j] * pe_st;",
                           "const double* prow = kv + b * kv_sb + set[j] * kv_st;"),
    "lse_without_log": ("m + log(denom)", "m + denom"),
    "head_stride_q_pe": ("q_pe + (b * H + h) * Dr", "q_pe + (b * H) * Dr"),
}


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(src), "-lm"])
    return oracle.load(str(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(tmp_path, name):
    lib = _build_mutant(tmp_path, name, *MUTANTS[name])

    def dec(**kw):
        return oracle.decode(**kw, lib=lib)

    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(dec)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


OUTPUT_PROJ_MUTANTS = {
    "transpose_wo": ("x[b * Din + i] * wo[o * Din + i]", "x[b * Din + i] * wo[i * Dout + o]"),
    "wo_drops_last_input": ("for (int64_t i = 0; i < Din; ++i) acc += x[b * Din + i]",
                            "for (int64_t i = 0; i + 1 < Din; ++i) acc += x[b * Din + i]"),
}


@pytest.mark.parametrize("name", sorted(OUTPUT_PROJ_MUTANTS))
def test_output_proj_mutant_fails_the_pin(tmp_path, name, monkeypatch):
    from tests import test_oracle_pins as tp
    lib = _build_mutant(tmp_path, name, *OUTPUT_PROJ_MUTANTS[name])
    real = oracle.output_proj
    monkeypatch.setattr(oracle, "output_proj", lambda x, wo: real(x, wo, lib=lib))
    with pytest.raises(AssertionError):
        tp.test_output_proj_brute_force()


PREFILL_MUTANTS = {
    "prefill_causal_excludes_diagonal": ("if (row[j] >= 0 && row[j] <= s) mark[row[j]] = 1;",
                                         "if (row[j] >= 0 && row[j] < s) mark[row[j]] = 1;"),
    "prefill_rotary_of_query_position": ("const double* kr = pe + b * pe_sb + t * pe_st;",
                                         "const double* kr = pe + b * pe_sb + s * pe_st;"),
    "prefill_values_from_w_uk": ("acc += w_uv[d * Dc + j] * c[j];", "acc += w_uk[d * Dc + j] * c[j];"),
    "prefill_drop_scale": ("sc[t] = acc * scale;", "sc[t] = acc;"),
    "prefill_transpose_w_uk": ("acc += w_uk[d * Dc + j] * c[j];", "acc += w_uk[j * Dn + d] * c[j];"),
    "prefill_no_causal_mask": ("for (int64_t t = 0; t <= s; ++t) mark[t] = (unsigned char)1;",
                               "for (int64_t t = 0; t < T; ++t) mark[t] = (unsigned char)1;"),
}


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_prefill_mutant_fails_a_pin(tmp_path, name):
    from tests import pins_prefill
    lib = _build_mutant(tmp_path, name, *PREFILL_MUTANTS[name])

    def pre(**kw):
        return oracle.prefill(**kw, lib=lib)

    failed = []
    for pin in pins_prefill.PREFILL_PINS:
        try:
            pin(pre)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every prefill pin"
