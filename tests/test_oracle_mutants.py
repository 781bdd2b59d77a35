"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/oracle.c``, plants one mistake by replacing a piece
of its text (a dropped term, a wrong sign or index, a transposed operand, a
wrong rounding rule), builds the copy with gcc into a temporary directory, and
asserts that at least one pin rejects it.  The real oracle is never modified.
Mutants are chosen so that none reads or writes outside its buffers.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "eps_outside_root": ("sqrt(mean_sq + (double)eps)", "(sqrt(mean_sq) + (double)eps)"),
    "no_root": ("1.0 / sqrt(mean_sq + (double)eps)", "1.0 / (mean_sq + (double)eps)"),
    "sum_not_mean": ("sum_sq / (double)hidden", "sum_sq"),
    "mean_over_hidden_minus_one": ("sum_sq / (double)hidden", "sum_sq / (double)(hidden > 1 ? hidden - 1 : 1)"),
    "eps_dropped": ("mean_sq + (double)eps", "mean_sq"),
    "square_dropped": ("sum_sq += v * v;", "sum_sq += fabs(v);"),
    "weight_dropped": ("z[j] = value_at(x, row * hidden + j, dtype) * rstd * wj;",
                       "z[j] = value_at(x, row * hidden + j, dtype) * rstd;"),
    "weight_reversed": ("value_at(w, j, dtype)", "value_at(w, hidden - 1 - j, dtype)"),
    "weight_none_zero": ("w ? value_at(w, j, dtype) : 1.0", "w ? value_at(w, j, dtype) : 0.5"),
    "rope_sign_first": ("head[i] = a * c - b * s;", "head[i] = a * c + b * s;"),
    "rope_sign_second": ("head[i + half] = b * c + a * s;", "head[i + half] = b * c - a * s;"),
    "rope_cos_sin_swapped": ("double c = (double)cp[i];", "double c = (double)sp[i];"),
    "rope_halves_swapped": ("double a = head[i];        /* first half  */\n                double b = head[i + half]; /* second half */",
                            "double b = head[i];        /* first half  */\n                double a = head[i + half]; /* second half */"),
    "rope_pair_mirrored": ("double b = head[i + half]; /* second half */",
                           "double b = head[head_dim - 1 - i]; /* second half */"),
    "rope_position_div": ("const int64_t p = r % seq_len;", "const int64_t p = (r / seq_len) % seq_len;"),
    "rope_position_zero": ("const int64_t p = r % seq_len;", "const int64_t p = 0;"),
    "rope_rounded_input": ("double a = head[i];        /* first half  */",
                           "double a = (double)(float)head[i]; /* first half  */"),
    "mag_signed": ("m[i] = fabs(a * c) + fabs(b * s);", "m[i] = fabs(a * c - b * s);"),
    "rope_il_sign_first": ("head[2 * i] = a * c - b * s;", "head[2 * i] = a * c + b * s;"),
    "rope_il_sign_second": ("head[2 * i + 1] = b * c + a * s;", "head[2 * i + 1] = b * c - a * s;"),
    "rope_il_table_reversed": ("double c = (double)cp[i];\n                double s = (double)sp[i];\n                head[2 * i]",
                               "double c = (double)cp[half - 1 - i];\n                double s = (double)sp[half - 1 - i];\n                head[2 * i]"),
    "rope_il_pairs_swapped": ("double a = head[2 * i];     /* even element */\n                double b = head[2 * i + 1]; /* odd element  */",
                              "double b = head[2 * i];     /* even element */\n                double a = head[2 * i + 1]; /* odd element  */"),
    "rope_il_mag_signed": ("m[2 * i] = fabs(a * c) + fabs(b * s);", "m[2 * i] = fabs(a * c - b * s);"),
    "adaln_scale_not_plus_one": ("double modulated = yr[j] * (1.0 + sc);", "double modulated = yr[j] * sc;"),
    "adaln_shift_subtracted": ("yr[j] = modulated + sh;", "yr[j] = modulated - sh;"),
    "adaln_shift_dropped": ("yr[j] = modulated + sh;", "yr[j] = modulated;"),
    "adaln_shift_scaled": ("yr[j] = modulated + sh;", "yr[j] = modulated + sh * (1.0 + sc);"),
    "adaln_mag_signed": ("mag[r * hidden + j] = fabs(modulated) + fabs(sh);", "mag[r * hidden + j] = fabs(modulated + sh);"),
    "adaln_sample_mod": ("const int64_t b = r / rows_per_sample;", "const int64_t b = r % rows_per_sample % (rows / rows_per_sample > 0 ? rows / rows_per_sample : 1);"),
    "adaln_scale_transposed": ("double sc = scale ? value_at(scale, b * hidden + j, dtype) : 0.0;",
                               "double sc = scale ? value_at(scale, b * hidden + (hidden - 1 - j), dtype) : 0.0;"),
    "f16_bias_14": ("ldexp((double)(1024 + fraction), exponent - 25)", "ldexp((double)(1024 + fraction), exponent - 24)"),
    "f16_subnormal_scale": ("v = ldexp((double)fraction, -24);", "v = ldexp((double)fraction, -25);"),
    "f16_sign_dropped": ("return sign ? -v : v;", "return v;"),
    "f16_overflow_at_max": ("if (a >= 65520.0)", "if (a >= 65504.0)"),
    "f16_truncate": ("double units = nearbyint(ldexp(a, 10 - e));", "double units = floor(ldexp(a, 10 - e));"),
    "f16_ties_away": ("double units = nearbyint(ldexp(a, 10 - e));", "double units = round(ldexp(a, 10 - e));"),
    "f16_no_subnormal_floor": ("    if (a == 0.0 || e < -14)\n        e = -14;", "    if (a == 0.0)\n        e = -14;"),
    "decode_f32_as_bf16": ("    return (double)((const float *)base)[i];", "    return bf16_value(((const uint16_t *)base)[i]);"),
    "bf16_ties_away": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    "bf16_truncate": ("kept += 1u;", "kept += 0u;"),
    "bf16_ties_odd": ("(kept & 1u))", "!(kept & 1u))"),
    "bf16_nan_not_quiet": ("return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);"),
    "round_skips_f32": ("float f = (float)y[i];", "float f = (float)(y[i] * (1.0 + 0x1p-20));"),
}


def _first_failing_pin(o):
    for pin in PINS:
        try:
            pin(o)
        except AssertionError:
            return pin.__name__
        except (ValueError, FloatingPointError, OverflowError, ZeroDivisionError, ArithmeticError):
            return pin.__name__
    return None


def test_real_oracle_passes_every_pin():
    assert _first_failing_pin(oracle.Oracle()) is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found in oracle.c"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    caught = _first_failing_pin(oracle.Oracle(lib))
    assert caught is not None, f"no pin rejects the planted mistake {name}"
