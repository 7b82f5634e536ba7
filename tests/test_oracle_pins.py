"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

from oracle import spc_oracle as O
from tests import pins


def test_scores_closed_form():
    pins.check_scores_closed_form(O.retrieval_scores)


def test_scores_zero_query_is_uniform():
    pins.check_scores_zero_query_uniform(O.retrieval_scores)


def test_scores_ignore_positions_past_length():
    pins.check_scores_length_masking(O.retrieval_scores)


def test_scores_match_library_attention_weights():
    pins.check_scores_vs_library(O.retrieval_scores)


def test_group_max_equals_per_head_max():
    pins.check_group_max_is_max_of_per_head(O.retrieval_scores, O.group_scores)


def test_group_modes_mha_mqa():
    pins.check_group_modes(O.group_scores)


def test_topk_bruteforce_tiny():
    pins.check_topk_bruteforce(O.topk_select)


def test_topk_python_sorted():
    pins.check_topk_python_sorted(O.topk_select)


def test_topk_edge_cases():
    pins.check_topk_edge_cases(O.topk_select)


def test_plan_worked_example_from_pages():
    pins.check_plan_worked_example(O.elastic_plan)


def test_plan_invariants():
    pins.check_plan_invariants(O.elastic_plan)


def test_plan_cold_repeat_growth():
    pins.check_plan_cold_repeat_growth(O.elastic_plan)


def test_copy_moves_rows_to_slots():
    pins.check_copy(O.elastic_copy, O.elastic_plan)


def test_attention_full_budget_is_dense_attention():
    pins.check_attention_full_budget(O.topk_select, O.sparse_decode_layer)


def test_attention_subset_matches_masked_library_attention():
    pins.check_attention_subset_vs_masked_library(O.sparse_attention)


def test_attention_special_cases():
    pins.check_attention_special_cases(O.sparse_attention)


def test_mla_literal_expansion_matches_absorbed_form():
    pins.check_mla_literal_vs_absorbed(O.mla_sparse_attention, O.mla_retrieval_scores)


def test_bf16_rounding_ties_to_even():
    from oracle.front import to_bf16_bits
    pins.check_round_bf16(O.round_bf16, to_bf16_bits)


def test_mla_expansion_stored_in_bf16_is_exact_on_integers():
    pins.check_mla_expand_exact(O.mla_expand_rows)


def test_kv_cache_size_matches_pages():
    pins.check_kv_cache_size(O.kv_cache_bytes)


def test_bf16_widening_exact():
    import numpy as np
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = O.to_f64(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625                      # 0x4049: 1.5703125 * 2
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127    # largest finite bf16
    assert vals[5] == 2.0 ** -133                   # smallest subnormal bf16


def test_offload_thresholds_worked_instance():
    pins.check_offload_golden(O.offload_thresholds, O.offloaded_layers)


def test_offload_thresholds_are_first_lengths_that_do_not_fit():
    pins.check_offload_invariants(O.offload_thresholds, O.memory_bytes)


def test_plan_lag1_worked_example():
    pins.check_plan_lag1_worked_example(O.elastic_plan_lag1)


def test_plan_lag1_reduces_to_the_blog_loop_plan():
    pins.check_plan_lag1_reduces_to_lag0(O.elastic_plan_lag1, O.elastic_plan)


def test_plan_lag1_invariants():
    pins.check_plan_lag1_invariants(O.elastic_plan_lag1)
