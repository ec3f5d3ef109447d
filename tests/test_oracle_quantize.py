"""Oracle pins: phase projection, axis scales, residual stages ("Step 2", "Step 3")."""
import numpy as np

import oracle
import pins


def test_project_bruteforce_with_ties():
    pins.check_project_bruteforce(oracle.project)


def test_project_nearest_by_angle():
    pins.check_project_angle(oracle.project)


def test_project_golden():
    pins.check_project_golden(oracle.project)


def test_ordered_sum_golden():
    pins.check_ordered_sum_golden(oracle.ordered_row_sum)


def test_ordered_sum_exact_on_integers():
    pins.check_ordered_sum_exact(oracle.ordered_row_sum)


def test_quantize_hand_worked():
    pins.check_quantize_hand(oracle.quantize, oracle.unsplit)


def test_least_squares_identity():
    pins.check_ls_identity(oracle.quantize, oracle.split, oracle.dequantize)


def test_residual_norm_nonincreasing():
    pins.check_norm_nonincreasing(oracle.quantize)


def test_codes_maximize_score_each_stage():
    pins.check_codes_maximize_score(oracle.quantize, oracle.split, oracle.dequantize)


def test_idempotent_on_representable_rows():
    pins.check_idempotent(oracle.quantize, oracle.unsplit)


def test_empty_axis_scale_is_zero():
    pins.check_empty_axis(oracle.quantize, oracle.unsplit)


def test_scales32_are_rne_of_scales64():
    R = (np.random.default_rng(0).standard_normal((32, 128)) * 0.02).astype(np.float32)
    _, s32, s64, _ = oracle.quantize(R, 3)
    assert s32.dtype == np.float32
    assert np.array_equal(s32, s64.astype(np.float32))


def test_dequantize_real_routes():
    pins.check_dequantize_real(oracle.dequantize_real, oracle.gemv_ref)


def test_per_tensor_scales():
    pins.check_per_tensor_scales(oracle.quantize, oracle.split)


def test_per_tensor_order():
    pins.check_per_tensor_order(oracle.quantize)
