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


# ---- the neighbours (output head, activation quantiser, block scales) ----

import test_oracle_neighbours as nbr  # noqa: E402

NEIGHBOUR_CHECKS = [
    nbr.test_quantize_hand_worked,
    nbr.test_quantize_special_tokens,
    lambda: [nbr.test_quantize_invariants(s) for s in range(3)],
    nbr.test_quantize_power_of_two_scaling,
    nbr.test_head_hand_worked,
    nbr.test_head_int_to_float_rounding,
    lambda: nbr.test_head_against_integer_matmul(3, 1000),
    nbr.test_head_overflow_reported,
    lambda: nbr.test_one_block_is_the_per_row_layer(100),
    lambda: nbr.test_blocked_against_integer_sums(1000, 128),
    nbr.test_blocked_equal_scales_reduce_to_row_scale,
]

NEIGHBOUR_MUTANTS = {
    "quant_range_not_widened": ("float lo = 0.0f, hi = 0.0f;", "float lo = r[0], hi = r[0];"),
    "quant_round_half_away": ("int32_t v = (int32_t)rintf(r[j] / s) + zm;",
                              "int32_t v = (int32_t)roundf(r[j] / s) + zm;"),
    "quant_256_steps": ("float s = (hi - lo) / 255.0f;", "float s = (hi - lo) / 256.0f;"),
    "quant_zero_point_sign": ("const int32_t zm = -128 - (int32_t)rintf(lo / s);",
                              "const int32_t zm = -128 + (int32_t)rintf(lo / s);"),
    "head_rowsum_skips_last": ("for (int64_t j = 0; j < K; ++j) s += W[i * ldw + j];",
                               "for (int64_t j = 0; j + 1 < K; ++j) s += W[i * ldw + j];"),
    "head_zero_point_dropped": ("const int64_t a = sum - (int64_t)rowsum[i] * (int64_t)z[m];",
                                "const int64_t a = sum;"),
    "head_single_rounding": ("float t = s_row[i] * fa;\n        y32[m * ldy + i] = t * s_act[m];",
                             "y32[m * ldy + i] = (float)((double)s_row[i] * (double)a * (double)s_act[m]);"
                             " (void)fa;"),
    "block_rowsum_overlaps": ("for (int64_t j = b * B; j < K && j < (b + 1) * B; ++j) s += w[i * ldw + j];",
                              "for (int64_t j = b * B; j < K && j <= (b + 1) * B; ++j) s += w[i * ldw + j];"),
    "block_scale_of_first_block": ("const float sb = s_b[i * nb + b];", "const float sb = s_b[i * nb];"),
    "block_zero_point_dropped": ("const int64_t a = sum - (int64_t)z[m] * (int64_t)rowsum_b[i * nb + b];",
                                 "const int64_t a = sum;"),
    "block_act_scale_dropped": ("if (y64) y64[m * ldy + i] = exact * (double)s_act[m];",
                                "if (y64) y64[m * ldy + i] = exact;"),
}


@pytest.mark.parametrize("name", sorted(NEIGHBOUR_MUTANTS))
def test_neighbour_pins_catch_mutant(name, tmp_path, monkeypatch):
    old, new = NEIGHBOUR_MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=path, out=os.path.join(str(tmp_path), "libmut.so")))
    monkeypatch.setattr(oracle, "_lib", lib)  # the neighbour pins use the default library
    caught = 0
    for check in NEIGHBOUR_CHECKS:
        try:
            check()
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:
            caught += 1
    assert caught, "no pin caught mutant %s" % name


# ---- the 1.6-bit layout (five weights per byte) ----

from test_oracle_packed5 import PACK5_CHECKS  # noqa: E402

PACK5_MUTANTS = {
    "pack5_digit_order_reversed": ("v += (unsigned)(wv + 1) * kPlace5[d];",
                                   "v += (unsigned)(wv + 1) * kPlace5[4 - d];"),
    "pack5_rounds_down": ("row[p] = (uint8_t)((256u * v + 242u) / 243u);",
                          "row[p] = (uint8_t)((256u * v) / 243u);"),
    "pack5_padding_minus_one": ("        int wv = 0;\n        if (j < K) {",
                                "        int wv = -1;\n        if (j < K) {"),
    "pack5_rowsum_skips_minus": ("          sum += wv;\n", "          sum += (wv > 0) ? wv : 0;\n"),
    "decode5_rounds_up": ("unsigned v = (243u * row[byte5_of(j)]) / 256u;",
                          "unsigned v = (243u * row[byte5_of(j)] + 255u) / 256u;"),
    "layout5_bytes_swapped": ("static int64_t byte5_of(int64_t j) { return 4 * (j / 20) + j % 4; }",
                              "static int64_t byte5_of(int64_t j) { return 4 * (j / 20) + 3 - j % 4; }"),
    "pack5_column_map_transposed": ("int64_t j = 20 * (p / 4) + 4 * d + p % 4;",
                                    "int64_t j = 20 * (p / 4) + 5 * (p % 4) + d;"),
    "linear5_zero_point_dropped": ("const int64_t a = dot - (int64_t)rowsum[i] * (int64_t)z[m];",
                                   "const int64_t a = dot;"),
    "linear5_epilogue_order": ("float prod = s_row[i] * (float)a; /* exact conversion, then round */\n"
                               "        y32[m * ldy + i] = prod * s_act[m];",
                               "float prod = (float)a * s_act[m];\n"
                               "        y32[m * ldy + i] = prod * s_row[i];"),
    "linear5_overflow_unchecked": ("      if (a >= limit || a <= -limit) {\n#pragma omp critical\n"
                                   "        if (status == ORACLE_OK) status = ORACLE_OVERFLOW;",
                                   "      if (0) {\n#pragma omp critical\n"
                                   "        if (status == ORACLE_OK) status = ORACLE_OVERFLOW;"),
}


@pytest.mark.parametrize("name", sorted(PACK5_MUTANTS))
def test_packed5_pins_catch_mutant(name, tmp_path):
    old, new = PACK5_MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=path, out=os.path.join(str(tmp_path), "libmut.so")))
    caught = []
    for check in PACK5_CHECKS:
        try:
            check(lib)
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:
            caught.append(check.__name__)
    assert caught, "no pin caught mutant %s" % name


# ---- the weight quantiser ----

from test_oracle_wquant import WQUANT_CHECKS  # noqa: E402

WQUANT_MUTANTS = {
    "wquant_full_block_count": ("const float scale = (float)(total / (double)(j1 - j0));",
                                "const float scale = (float)(total / (double)B);"),
    "wquant_signed_sum": ("total += fabs((double)row[j]);", "total += (double)row[j];"),
    "wquant_round_half_away": ("state = rintf(ratio);", "state = roundf(ratio);"),
    "wquant_no_clamp": ("if (ratio > 1.0f) ratio = 1.0f;", "if (ratio > 9.0f) ratio = 1.0f;"),
    "wquant_blocks_shifted": ("const int64_t j0 = b * B, j1 = (j0 + B < K) ? j0 + B : K;",
                              "const int64_t j0 = b * B + (b > 0), j1 = (j0 + B < K) ? j0 + B : K;"),
    "wquant_fp32_sum": ("double total = 0.0;\n      for (int64_t j = j0; j < j1; ++j) total += fabs((double)row[j]);",
                        "float total = 0.0f;\n      for (int64_t j = j0; j < j1; ++j) total += fabsf(row[j]);"),
}


@pytest.mark.parametrize("name", sorted(WQUANT_MUTANTS))
def test_wquant_pins_catch_mutant(name, tmp_path):
    old, new = WQUANT_MUTANTS[name]
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found once: %s" % name
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(force=True, src=path, out=os.path.join(str(tmp_path), "libmut.so")))
    caught = []
    for check in WQUANT_CHECKS:
        try:
            check(lib)
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:
            caught.append(check.__name__)
    assert caught, "no pin caught mutant %s" % name
