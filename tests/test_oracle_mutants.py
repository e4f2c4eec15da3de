"""Planted mistakes: copies of the oracle's C source with one plausible error
each (a dropped term, a wrong sign or index, a swapped operand, a wrong
rounding) must fail at least one pin.  CPU only; the mutants are built with
gcc into a temporary directory and never leave this test."""
import os
import subprocess

import pytest

import oracle_pins as P
from oracle import build as B
from oracle import oracle as O

MUTANTS = [
    ("variance_divides_by_H_minus_1", "double var = ss / (double)H;", "double var = ss / (double)(H - 1);"),
    ("mean_divides_by_H_plus_1", "mean = sum / (double)H;", "mean = sum / (double)(H + 1);"),
    ("bias_dropped", "a = a + load_t(J->bias, c, J->dtype);", "a = a;"),
    ("sum_rounded_once_from_binary64",
     "a = a + load_t(J->bias, c, J->dtype);",
     "a = (float)((double)load_t(J->input, i * H + c, J->dtype) + (double)load_t(J->skip, j * H + c, J->dtype)"
     " + (double)load_t(J->bias, c, J->dtype));"),
    ("residual_stored_before_bias",
     "            if (J->bias)\n                a = a + load_t(J->bias, c, J->dtype);\n            s[c] = a;\n"
     "            if (J->residual_out)\n                store_t(J->residual_out, i * H + c, a, J->dtype);",
     "            if (J->residual_out)\n                store_t(J->residual_out, i * H + c, a, J->dtype);\n"
     "            if (J->bias)\n                a = a + load_t(J->bias, c, J->dtype);\n            s[c] = a;"),
    ("sign_flipped", "((double)s[c] - mean) / denom", "(mean - (double)s[c]) / denom"),
    ("eps_outside_sqrt", "sqrt(var + J->eps)", "(sqrt(var) + J->eps)"),
    ("eps_ignored", "sqrt(var + J->eps)", "sqrt(var)"),
    ("mean_not_subtracted_in_variance", "double d = (double)s[c] - mean;", "double d = (double)s[c];"),
    ("variance_deviation_in_binary32", "double d = (double)s[c] - mean;", "double d = (float)((double)s[c] - mean);"),
    ("broadcast_ignores_row_offset", "(J->row_offset + i) % J->skip_rows", "i % J->skip_rows"),
    ("broadcast_reads_first_skip_row", "(J->row_offset + i) % J->skip_rows", "0"),
    ("gamma_beta_swapped", "* g + b;", "* b + g;"),
    ("beta_ignored", "J->beta ? (double)load_t(J->beta, c, J->dtype) : 0.0", "0.0"),
    ("gamma_columns_reversed", "load_t(J->gamma, c, J->dtype)", "load_t(J->gamma, J->hidden - 1 - c, J->dtype)"),
    ("f16_truncates", "if (rem > half || (rem == half && (q & 1u)))", "if (0)"),
    ("f16_ties_away_from_zero", "(rem == half && (q & 1u))", "(rem == half)"),
    ("f16_flushes_subnormals", "if (shift > 24)", "if (shift > 0)"),
    ("f16_decode_subnormal_scale", "ldexpf((float)m, -24)", "ldexpf((float)m, -23)"),
    ("bias_add_skip_first", "float a = xv + bv;\n            a = a + sv;", "float a = xv + sv;\n            a = a + bv;"),
    ("skipln_bias_joins_skip_first",
     "            float a = load_t(J->input, i * H + c, J->dtype) + load_t(J->skip, j * H + c, J->dtype);\n"
     "            if (J->bias)\n                a = a + load_t(J->bias, c, J->dtype);",
     "            float a = load_t(J->skip, j * H + c, J->dtype);\n"
     "            if (J->bias)\n                a = a + load_t(J->bias, c, J->dtype);\n"
     "            a = load_t(J->input, i * H + c, J->dtype) + a;"),
    ("rms_keeps_mean", "if (!J->simplified) {", "if (1) {"),
    ("softmax_inner_outer_swapped", "const int64_t j = inner ? r / repeat : r % bias_rows;",
     "const int64_t j = inner ? r % bias_rows : r / repeat;"),
    ("softmax_max_not_subtracted", "sum += exp(z[c] - m);", "sum += exp(z[c]);"),
    ("softmax_bias_ignored", "+ load_t(bias, j * block_size + c, dtype);", ";"),
    ("softmax_max_from_first_column", "if (z[c] > m)", "if (c == 0)"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def _build_mutant(d, name, old, new):
    src = open(B.SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found in the oracle source"
    path = os.path.join(str(d), f"{name}.c")
    with open(path, "w") as fh:
        fh.write(src.replace(old, new))
    lib = os.path.join(str(d), f"lib{name}.so")
    cmd = [a for a in B.CMD if a not in ("-Werror",)]
    cmd[cmd.index(B.SRC)] = path
    subprocess.run(cmd + [lib, "-lm"], check=True, capture_output=True)
    return lib


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(mutant_dir, name, old, new):
    lib = _build_mutant(mutant_dir, name, old, new)
    O.use(lib)
    try:
        caught = []
        for check in P.ALL_CHECKS:
            try:
                check()
            except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
                caught.append((check.__name__, str(e)[:80]))
                break
    finally:
        O.use(None)
    assert caught, f"no pin catches the planted mistake {name}"


# Mistakes in the grouping of the binary32 adds must be caught by the
# hand-derived golden rows themselves, not only by checks whose expected sum
# is formed in numpy in the oracle's own order.
GOLDEN_CATCHES = {
    "bias_add_skip_first": P.check_bias_add_hand_rows,
    "skipln_bias_joins_skip_first": P.check_hand_rows,
    "residual_stored_before_bias": P.check_hand_rows,
}


@pytest.mark.parametrize("name", sorted(GOLDEN_CATCHES))
def test_add_order_mistake_fails_a_golden_row(mutant_dir, name):
    old, new = next((o, n) for m, o, n in MUTANTS if m == name)
    lib = _build_mutant(mutant_dir, name + "_golden", old, new)
    O.use(lib)
    try:
        with pytest.raises(AssertionError):
            GOLDEN_CATCHES[name]()
    finally:
        O.use(None)
