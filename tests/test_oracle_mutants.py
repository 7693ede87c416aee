"""Plant plausible mistakes in a copy of the oracle; the pins must catch each.

Every mutant is a one-spot textual edit of ``oracle/serac_oracle.c``,
compiled into a temporary library on the CPU.  The real oracle is never
modified.  A mutant that passes every pin means the pins have a blind spot.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "row_tie_keeps_last_column": ("if (s > best) {\n            second = best;",
                                  "if (s >= best) {\n            second = best;"),
    "second_without_multiplicity": ("} else if (s > second) {",
                                    "} else if (s > second && s != best) {"),
    "second_not_demoted": ("            second = best;\n            best = s;",
                           "            best = s;"),
    "row_seed_below_zero": ("int32_t best = 0, idx = -1, second = 0;",
                            "int32_t best = -1, idx = -1, second = -1;"),
    "row_index_off_by_one": ("            idx = j;\n", "            idx = j + 1;\n"),
    "col_tie_keeps_last_row": ("if (s > best) {\n                        best = s;",
                               "if (s >= best) {\n                        best = s;"),
    "col_seed_below_zero": ("col_best[2 * j] = 0;", "col_best[2 * j] = -1;"),
    "dot_drops_first_term": ("for (int k = 0; k < DIM; ++k)",
                             "for (int k = 1; k < DIM; ++k)"),
    "dot_transposed_operand": ("srow[j] = dot(a, B + (size_t)j * DIM);",
                               "srow[j] = dot(a, B + (size_t)((j + 1) % nB) * DIM);"),
    "ratio_not_strict": ("if (!(d1 < max_ratio * d2))", "if (!(d1 <= max_ratio * d2))"),
    "ratio_inverted": ("if (!(d1 < max_ratio * d2))", "if (!(d2 < max_ratio * d1))"),
    "distance_not_inclusive": ("if (!(d1 <= max_distance))", "if (!(d1 < max_distance))"),
    "cosine_wrong_norm": ("(double)s / (double)NORM2", "(double)s / 262143.0"),
    "cosine_not_clamped": ("(s >= NORM2) ? 1.0 :", "0 ? 1.0 :"),
    "cross_check_ignored": ("if (cross_check && colidx_of_best != i)", "if (0)"),
    "sym_column_gate_dropped": (
        "if (!oracle_accept(j, cbest, ci, csecond, -1, max_ratio, max_distance, 0))",
        "if (0)"),
    "sym_mutual_check_dropped": ("if (ci != i)\n                continue;", "if (0)\n                continue;"),
    "sym_column_second_from_row": ("csecond = col[3 * j + 2];", "csecond = second;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    L = oracle.load(so)
    failed = []
    for pin in PINS:
        try:
            pin(L)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
