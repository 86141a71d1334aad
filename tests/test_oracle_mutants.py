"""Plants plausible mistakes in a copy of the oracle's C source and checks the pins catch each.

Every mutant is a one-place edit of msa_oracle.c (a dropped term, a wrong sign,
a transposed or mis-indexed operand, an unmasked tail, a pinning or ordering
slip), built with the same compiler flags into a temporary library. Each edit
keeps every memory access in bounds. A mutant that no pin rejects would mean
the pins do not pin that part of the oracle.
"""
import os

import pytest

import oracle
from oracle.build import SOURCE, build

from test_oracle_pins import PINS

MUTANTS = {
    "dropped_dim": ("for (int d = 0; d < OR_DIM; ++d) s +=", "for (int d = 1; d < OR_DIM; ++d) s +="),
    "wrong_sign": ("s += widen_bf16(qh[d]) * kt[d];", "s -= widen_bf16(qh[d]) * kt[d];"),
    "transposed_page": ("kt[d] = widen_bf16(k16[d]);",
                        "kt[d] = widen_bf16(((const uint16_t *)k_cache)[(page * OR_BLOCK + d) * OR_DIM + t]);"),
    "head_index": ("q + ((int64_t)b * OR_HEADS + h) * OR_DIM",
                   "q + ((int64_t)b * OR_HEADS + (OR_HEADS - 1 - h)) * OR_DIM"),
    "tail_unmasked": ("if (valid > OR_BLOCK) valid = OR_BLOCK;", "valid = OR_BLOCK;"),
    "logical_order": ("block_table[(int64_t)b * bt_stride + j];\n            if (page < 0",
                      "block_table[(int64_t)b * bt_stride + (nb - 1 - j)];\n            if (page < 0"),
    "max_seeded_zero": ("for (int h = 0; h < OR_HEADS; ++h) best[h] = -INFINITY;",
                        "for (int h = 0; h < OR_HEADS; ++h) best[h] = 0.0;"),
    "recent_pin_off_by_one": ("(j >= nb - n_local)", "(j > nb - n_local)"),
    "init_pin_off_by_one": ("c[j].pinned = (j < n_init)", "c[j].pinned = (j <= n_init)"),
    "pins_not_first": ("if (a->pinned != b->pinned) return a->pinned ? -1 : 1;", ""),
    "ties_descending": ("return (a->id < b->id) ? -1 : (a->id > b->id);",
                        "return (a->id > b->id) ? -1 : (a->id < b->id);"),
    "ascending_scores": ("if (a->score > b->score) return -1;\n    if (a->score < b->score) return 1;",
                         "if (a->score < b->score) return -1;\n    if (a->score > b->score) return 1;"),
    "pad_id_zero": ("out_ids[bh * topk + i] = i < m ? c[i].id : -1;",
                    "out_ids[bh * topk + i] = i < m ? c[i].id : 0;"),
    "short_row_truncated": ("int64_t m = nb < topk ? nb : topk;",
                            "int64_t m = nb < topk ? nb - 1 : topk;"),
    "pages_not_sorted": ("qsort(sel, (size_t)n, sizeof(int32_t), cmp_int);", ""),
    "page_offset": ("row[i * 8 + t] = (int32_t)(uint32_t)(page * 8 + t);",
                    "row[i * 8 + t] = (int32_t)(uint32_t)(page * 8 + t + 1);"),
    "ids_past_row_kept": ("if (j >= 0 && j < nb) sel[n++] = j;", "if (j >= 0 && j < max_blocks) sel[n++] = j;"),
    "repeats_dropped": ("if (j >= 0 && j < nb) sel[n++] = j;",
                        "if (j >= 0 && j < nb && (n == 0 || sel[n - 1] != j)) sel[n++] = j;"),
    "causal_reversed": ("int64_t L = row_len(seq_lens, b, max_blocks) - (qlen - 1 - p);",
                        "int64_t L = row_len(seq_lens, b, max_blocks) - p;"),
    "causal_off_by_one": ("int64_t L = row_len(seq_lens, b, max_blocks) - (qlen - 1 - p);",
                          "int64_t L = row_len(seq_lens, b, max_blocks) - (qlen - p);"),
    "positions_swapped": ("q + ((size_t)b * qlen + p) * OR_HEADS * OR_DIM",
                          "q + ((size_t)b * qlen + (qlen - 1 - p)) * OR_HEADS * OR_DIM"),
    "e4m3_bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3_sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "fp8_scale_dropped": ("kt[d] = k_scale * widen_e4m3(k8[d]);", "kt[d] = widen_e4m3(k8[d]);"),
    "tokens_full_blocks": ("count += valid > OR_BLOCK ? OR_BLOCK : valid;", "count += OR_BLOCK;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SOURCE).read()
    assert src.count(before) == 1, f"mutation site for {name} not unique or missing"
    path = tmp_path / "msa_oracle_mutant.c"
    path.write_text(src.replace(before, after))
    lib = build(src=str(path), out=str(tmp_path / f"libmutant_{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for check in PINS:
        try:
            check(orc)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin rejects the {name} mutant"


def test_unmutated_copy_passes_every_pin(tmp_path):
    # The same build route as the mutants, without an edit, passes all pins.
    path = tmp_path / "msa_oracle_copy.c"
    path.write_text(open(SOURCE).read())
    orc = oracle.Oracle(build(src=str(path), out=str(tmp_path / "libcopy.so")))
    for check in PINS:
        check(orc)
