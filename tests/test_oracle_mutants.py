"""The oracle's pins must catch plausible mistakes.

Each case plants one slip in a temporary copy of the oracle's C source (on
the CPU; the real oracle is untouched), builds it, and runs every pin check
from ``test_oracle_pins``: at least one must fail.
"""
import os

import pytest

import oracle
from test_oracle_pins import ALL_CHECKS

MUTANTS = {
    "plus_minus_swapped": ("write_code(row, j, (unsigned)(v + 1));",
                           "write_code(row, j, (unsigned)(1 - v));"),
    "layout_transposed": ("static int64_t field_byte(int64_t j) { return 4 * (j / 16) + j % 4; }\n"
                          "static int field_shift(int64_t j) { return 2 * (int)((j % 16) / 4); }",
                          "static int64_t field_byte(int64_t j) { return 4 * (j / 16) + (j % 16) / 4; }\n"
                          "static int field_shift(int64_t j) { return 2 * (int)(j % 4); }"),
    "padding_not_zero_weight": ("memset(row, 0x55, (size_t)ld);", "memset(row, 0x00, (size_t)ld);"),
    "zero_point_sign": ("int64_t a = sum - (int64_t)z[m] * (int64_t)rowsum[i];",
                        "int64_t a = sum + (int64_t)z[m] * (int64_t)rowsum[i];"),
    "zero_point_dropped": ("int64_t a = sum - (int64_t)z[m] * (int64_t)rowsum[i];",
                           "int64_t a = sum;"),
    "rowsum_counts_plus_only": ("      sum += v;\n", "      sum += (v > 0);\n"),
    "unpack_no_offset": ("w[i * ldw + j] = (int8_t)((int)c - 1);", "w[i * ldw + j] = (int8_t)((int)c);"),
    "last_column_dropped": ("if (wv > 0) sum += q[m * ldq + j];",
                            "if (wv > 0 && j + 1 < K) sum += q[m * ldq + j];"),
    "activation_reversed": ("if (wv > 0) sum += q[m * ldq + j];\n        else if (wv < 0) sum -= q[m * ldq + j];",
                            "if (wv > 0) sum += q[m * ldq + K - 1 - j];\n"
                            "        else if (wv < 0) sum -= q[m * ldq + K - 1 - j];"),
    "epilogue_order": ("float t = s_row[i] * fa;       /* first rounding  */\n"
                       "        y32[m * ldy + i] = t * s_act[m]; /* second rounding */",
                       "float t = fa * s_act[m];\n        y32[m * ldy + i] = t * s_row[i];"),
    "epilogue_single_rounding": ("y32[m * ldy + i] = t * s_act[m]; /* second rounding */",
                                 "y32[m * ldy + i] = (float)((double)s_row[i] * (double)fa"
                                 " * (double)s_act[m]); (void)t;"),
    "direct_zero_point_sign": ("((int64_t)q[m * ldq + j] - (int64_t)z[m])",
                               "((int64_t)q[m * ldq + j] + (int64_t)z[m])"),
    "overflow_unchecked": ("(a >= limit || a <= -limit) ? ORACLE_OVERFLOW : 0",
                           "0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=path, out=os.path.join(str(tmp_path), "libmut.so")))
    caught = []
    for check in ALL_CHECKS:
        try:
            check(lib)
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:  # AssertionError, ValueError, pytest's Failed
            caught.append(check.__name__)
    assert caught, "no pin caught mutant %s" % name
