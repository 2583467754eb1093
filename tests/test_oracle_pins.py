"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from tests import oracle_pins as P


def test_golden_single():
    P.pin_golden_single(oracle.lora_fwd, oracle.lora_bwd_dx_da, oracle.lora_bwd_db)


def test_fwd_dense_identity():
    P.pin_fwd_dense_identity(oracle.lora_fwd)


def test_fwd_special_cases():
    P.pin_fwd_special_cases(oracle.lora_fwd)


def test_bwd_finite_differences():
    P.pin_bwd_finite_differences(oracle.lora_fwd, oracle.lora_bwd_dx_da, oracle.lora_bwd_db)


def test_bwd_euler_identity():
    P.pin_bwd_euler(oracle.lora_fwd, oracle.lora_bwd_dx_da, oracle.lora_bwd_db)


def test_bwd_dense_chain_rule():
    P.pin_bwd_dense_chain(oracle.lora_bwd_dx_da, oracle.lora_bwd_db)


def test_single_brute_force():
    P.pin_single_brute_force(oracle.lora_fwd, oracle.lora_bwd_dx_da, oracle.lora_bwd_db)


def test_single_integer_exact():
    P.pin_single_integer_exact(oracle.lora_fwd, oracle.lora_bwd_dx_da, oracle.lora_bwd_db)


def test_golden_multi():
    P.pin_golden_multi(oracle.shrink, oracle.expand_fused, oracle.group_tokens)


def test_golden_gather():
    P.pin_golden_gather(oracle.gather_shrink)


def test_golden_grouping():
    P.pin_golden_grouping(oracle.group_tokens)


def test_multi_brute_force():
    P.pin_multi_brute_force(oracle.shrink, oracle.expand_fused)


def test_multi_reduces_to_single():
    P.pin_multi_reduces_to_single(oracle.lora_fwd, oracle.shrink, oracle.expand_fused)


def test_gather_is_onehot_shrink():
    P.pin_gather_is_onehot_shrink(oracle.gather_shrink, oracle.shrink)


def test_grouping_is_stable_sort():
    P.pin_grouping_is_stable_sort(oracle.group_tokens)


def test_golden_active():
    P.pin_golden_active(oracle.token_ranks, oracle.active_mask, oracle.group_tokens)


def test_active_mask():
    P.pin_active_mask(oracle.token_ranks, oracle.active_mask, oracle.group_tokens)


def test_golden_apply_linear():
    P.pin_golden_apply(oracle.apply_linear)


def test_apply_linear_brute_force():
    P.pin_apply_linear_brute(oracle.apply_linear)


def test_golden_bf16_widening():
    P.pin_golden_bf16(oracle.bf16_bits_to_f64)


def test_bf16_widening_closed_form():
    P.pin_bf16_closed_form(oracle.bf16_bits_to_f64)


def test_golden_bf16_rounding():
    P.pin_golden_bf16_round(oracle.round_to_bf16)


def test_bf16_rounding_grid():
    P.pin_bf16_round_grid(oracle.round_to_bf16, oracle.bf16_bits_to_f64)


def test_bf16_rounding_matches_torch_on_float32():
    P.pin_bf16_round_f32(oracle.round_to_bf16)


def test_apply_linear_is_shrink_then_expand():
    import numpy as np
    rng = np.random.default_rng(31)
    ts, ranks, x, a, b, sc, y0 = P._rand_multi(rng, 9, 4, (3, 2), 3, 2)
    h = oracle.shrink(x, a, ts, ranks, 2, 2)
    want = oracle.expand_fused(h, b, ts, ranks, sc, y0, (3, 2), 2)
    got = oracle.apply_linear(x, y0, a, b, ts, ranks, sc, (3, 2), 2)
    assert np.array_equal(got, want)


def test_token_subsets_match_full():
    """Computing only some rows (as the full-size parity tests do) gives the
    same rows as the full computation."""
    import numpy as np
    rng = np.random.default_rng(32)
    ts, ranks, x, a, b, sc, y0 = P._rand_multi(rng, 15, 6, (4, 3), 4, 3)
    sub = [14, 0, 7, 3]
    h_full = oracle.shrink(x, a, ts, ranks, 2, 3)
    h_sub = oracle.shrink(x, a, ts, ranks, 2, 3, tokens=sub)
    assert np.array_equal(h_full[sub], h_sub[sub])
    y_full = oracle.expand_fused(h_full, b, ts, ranks, sc, y0, (4, 3), 3)
    y_sub = oracle.expand_fused(h_full, b, ts, ranks, sc, y0, (4, 3), 3, tokens=sub)
    assert np.array_equal(y_full[sub], y_sub)


def test_rel_frobenius_basics():
    import numpy as np
    assert oracle.rel_frobenius([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert abs(oracle.rel_frobenius([3.0, 4.0], [0.0, 5.0]) - (np.sqrt(9 + 1) / 5)) < 1e-15
    assert oracle.rel_frobenius([0.0], [0.0]) == 0.0
    assert oracle.rel_frobenius([1e-30], [0.0]) == float("inf")
