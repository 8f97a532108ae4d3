"""The FP64 oracle against facts fixed outside it (CPU only)."""

import oracle
import oracle_pins as P


def test_nonabsorbed_identity():
    P.pin_nonabsorbed_identity(oracle.mla_decode_ref_f64)


def test_page_permutation_invariance():
    P.pin_page_permutation(oracle.mla_decode_ref)


def test_single_token():
    P.pin_single_token(oracle.mla_decode_ref)


def test_equal_scores():
    P.pin_equal_scores(oracle.mla_decode_ref_f64)


def test_causal_reductions():
    P.pin_causal_reductions(oracle.mla_decode_ref)


def test_combine_identity():
    P.pin_combine_identity(oracle.attend_rows, oracle.lse_combine_ref)


def test_bruteforce():
    P.pin_bruteforce(oracle.mla_decode_ref_f64)


def test_bounds():
    P.pin_bounds(oracle.mla_decode_ref)


def test_two_keys_by_hand():
    P.pin_two_keys(oracle.mla_decode_ref_f64)


def test_append_physical_view():
    P.pin_append_physical_view(oracle.kv_append_ref)


def test_append_round_trip():
    P.pin_append_round_trip(oracle.kv_append_ref)


def test_absorb_end_to_end():
    P.pin_absorb_end_to_end(oracle.absorb_q_ref, oracle.absorb_o_ref, oracle.mla_decode_ref_f64)


def test_absorb_selection():
    P.pin_absorb_selection(oracle.absorb_q_ref, oracle.absorb_o_ref)


def test_e4m3_table():
    P.pin_e4m3_table(oracle.e4m3_decode)


def test_e4m3_quantizer():
    P.pin_e4m3_quantizer(oracle.quantize_e4m3_rows, oracle.e4m3_decode)


def test_fp8_decode_matches_bf16():
    P.pin_fp8_decode_matches_bf16(oracle.mla_decode_fp8_ref, oracle.mla_decode_ref)


def test_e4m3_quantizer_bruteforce():
    P.pin_e4m3_quantizer_bruteforce(oracle.quantize_e4m3_rows, oracle.e4m3_decode)


def test_e4m3_exact_quotient():
    P.pin_e4m3_exact_quotient(oracle.quantize_e4m3_rows, oracle.e4m3_decode)


def test_append_fp8_physical_view():
    P.pin_append_fp8_physical_view(oracle.kv_append_fp8_ref, oracle.quantize_e4m3_rows)


def test_mha_bruteforce():
    P.pin_mha_bruteforce(oracle.mha_decode_ref)


def test_mha_grouping_and_invariants():
    P.pin_mha_grouping_and_invariants(oracle.mha_decode_ref)
