"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutant is the oracle's C source with one textual change, compiled on the
CPU into a temporary library.  The test fails if a mutant passes every pin,
which would mean the pins could not tell that mistake from the real thing.
"""
import os

import pytest

from oracle import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ts_oracle.c")

# (name, original, replacement[, original, replacement ...]) -- every original must
# occur in the source; the first occurrence is the one replaced.
MUTANTS = [
    ("sink_dropped_from_denominator",
     "double den = (sigma == -INFINITY) ? 0.0 : exp(sigma - m);", "double den = 0.0;"),
    ("sink_multiplied_by_scale",
     "const double sigma = sinks ? (double)sinks[h] : -INFINITY;",
     "const double sigma = sinks ? scale * (double)sinks[h] : -INFINITY;"),
    ("sink_sign_flipped",
     "const double sigma = sinks ? (double)sinks[h] : -INFINITY;",
     "const double sigma = sinks ? -(double)sinks[h] : -INFINITY;"),
    ("sink_given_a_value_row",
     "    den += w;\n",
     "    den += w;\n    if (j == jlo && sigma != -INFINITY)\n"
     "      for (int32_t d = 0; d < head_dim; ++d) acc[d] += exp(sigma - m) * bf16_to_double(vrow[d]);\n"),
    ("window_off_by_one_wide", "int64_t lo = i - (int64_t)window + 1;", "int64_t lo = i - (int64_t)window;"),
    ("window_off_by_one_narrow", "int64_t lo = i - (int64_t)window + 1;", "int64_t lo = i - (int64_t)window + 2;"),
    ("diagonal_excluded_pass1", "for (int64_t j = jlo; j <= i; ++j) {\n    const uint16_t* krow",
     "for (int64_t j = jlo; j < i; ++j) {\n    const uint16_t* krow"),
    ("gqa_mapping_modulo", "const int32_t g = h / G;", "const int32_t g = h % n_kv_heads;"),
    ("key_row_at_query_position", "k + ((s + j) * n_kv_heads + g)", "k + ((s + i) * n_kv_heads + g)"),
    ("value_operand_is_key", "const uint16_t* vrow = v +", "const uint16_t* vrow = k +"),
    ("scale_omitted", "z[j - jlo] = scale * dot;", "z[j - jlo] = dot;"),
    ("exponent_sign_flipped", "const double w = exp(z[j - jlo] - m);", "const double w = exp(m - z[j - jlo]);"),
    ("positions_not_relative_to_sequence",
     "one_row(q, k, v, sinks, s, t - s, h,", "one_row(q, k, v, sinks, 0, t, h,",
     # second site keeps the mutant memory-safe: rows now see up to T keys
     "double* z = (double*)malloc(sizeof(double) * (size_t)max_len);",
     "double* z = (double*)malloc(sizeof(double) * (size_t)T);"),
    ("denominator_misses_keys", "    den += w;\n", "    den += (j == i) ? w : 0.0;\n"),
    ("sink_share_unshifted", "*p_sink = (sigma == -INFINITY) ? 0.0 : exp(sigma - m) / den;",
     "*p_sink = (sigma == -INFINITY) ? 0.0 : exp(sigma) / den;"),
    ("bf16_widening_wrong_half", "uint32_t w = ((uint32_t)bits) << 16;", "uint32_t w = ((uint32_t)bits) << 15;"),
    # the selected-rows routine
    ("rows_start_of_previous_sequence",
     "seq_of_row(cu_seqlens, n_seqs, rows[n]);\n        const int64_t s = cu_seqlens[b];",
     "seq_of_row(cu_seqlens, n_seqs, rows[n]);\n        const int64_t s = cu_seqlens[b > 0 ? b - 1 : 0];",
     # keeps the mutant memory-safe: a row may now see more keys than its sequence holds
     "double* z = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));",
     "double* z = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));"),
    ("rows_output_in_reverse_order", "out + n * (int64_t)head_dim, NULL, NULL",
     "out + (n_rows - 1 - n) * (int64_t)head_dim, NULL, NULL"),
    ("rows_head_of_first_entry", "rows[n] - s, heads[n], n_q_heads", "rows[n] - s, heads[0], n_q_heads"),
    ("rows_query_one_position_early", "rows[n] - s, heads[n], n_q_heads",
     "rows[n] - s - (rows[n] > s), heads[n], n_q_heads"),
    # the paged-cache form
    ("cache_top_left_alignment",
     "const int64_t p = (int64_t)seqlens_k[b] - q_len + (t - cu_seqlens_q[b]);",
     "const int64_t p = t - cu_seqlens_q[b];"),
    ("cache_table_row_ignored", "const int32_t* pages = block_table + (int64_t)b * pages_per_seq;",
     "const int32_t* pages = block_table;"),
    ("cache_window_off_by_one", "const int64_t jlo = first_visible(p, window);",
     "const int64_t jlo = first_visible(p + 1, window);"),
    ("cache_value_from_key_cache", "const uint16_t* vrow = v_cache +", "const uint16_t* vrow = k_cache +"),
    ("cache_value_slot_shifted", "page_size + j % page_size) * n_kv_heads",
     "page_size + (j + 1) % page_size) * n_kv_heads"),
    ("cache_sink_dropped", "double den = sinks ? exp(sigma - m) : 0.0;", "double den = 0.0;"),
    ("cache_rows_without_keys_not_zero", "if (p < 0) return TS_ORACLE_OK;", "if (p < 0) p = 0;"),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mutant, tmp_path):
    name, edits = mutant[0], mutant[1:]
    mutated = open(SRC).read()
    for old, new in zip(edits[0::2], edits[1::2]):
        assert old in mutated, f"mutation site for {name} no longer exists in the oracle source"
        mutated = mutated.replace(old, new, 1)
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    lib_path = oracle.build(src=str(path), out=str(tmp_path / f"lib{name}.so"),
                            extra_flags=("-Wno-unused-parameter", "-Wno-unused-variable"))
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
