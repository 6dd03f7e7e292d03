"""The oracle against the pages' printed values, closed forms, brute force and invariants (CPU only)."""

import oracle
import oracle_checks as oc


def test_kv_size_formula_printed_values():
    oc.check_kv_formula(oracle.kv_bytes)
    assert oracle.kv_bytes_per_token(80, 64, 128, 2) == 2_621_440


def test_decode_bits_exact_values():
    oc.check_decode_bits(oracle.decode_bits)


def test_ref_decode_matches_token_by_token_bruteforce():
    oc.check_bruteforce(oracle.ref_decode, oracle.bruteforce_decode)


def test_closed_forms():
    oc.check_closed_forms(oracle.ref_decode)


def test_physical_placement_permutation_is_bitwise_invariant():
    oc.check_permutation_invariance(oracle.ref_decode)


def test_gqa_equals_mha_on_repeat_interleaved_kv():
    oc.check_gqa_equals_repeated_mha(oracle.ref_decode)


def test_output_in_convex_hull_of_values():
    oc.check_convex_hull(oracle.ref_decode)


def test_matches_library_sdpa_on_gathered_kv():
    oc.check_sdpa(oracle.ref_decode)


def test_worked_fork_refcount_example():
    oc.check_worked_example(oracle.RefPool)


def test_pool_error_conventions_and_all_or_nothing():
    oc.check_error_conventions(oracle.RefPool)


def test_slot_arithmetic_and_last_block_waste():
    oc.check_slot_arithmetic(oracle.RefPool)


def test_pool_random_walk_against_unpaged_model():
    for seed in range(4):
        oc.check_pool_against_unpaged_model(oracle.RefPool, oracle.apply_append, seed=seed)


def test_identical_histories_give_identical_bytes():
    oc.check_identical_histories_identical_bytes(oracle.RefPool, oracle.apply_append)


def test_rows_subset_equals_full():
    import numpy as np
    rng = np.random.default_rng(1)
    q, k, v, bt, sl = oc.random_paged_case(rng, 4, 4, 2, 8, 16, [3, 40, 0, 17], "bf16")
    full = oracle.ref_decode(q, k, v, bt, sl, 0.3, "bf16")
    part = oracle.ref_decode_rows(q, k, v, bt, sl, 0.3, "bf16", rows=[3, 1])
    assert np.array_equal(part, full[[3, 1]])
