"""Oracle pins: the multiplication-free widely-linear GEMV."""
import oracle
import pins


def test_gemv_hand_worked():
    pins.check_gemv_hand(oracle.gemv_ref)


def test_gemv_three_routes_and_stage_sum():
    pins.check_gemv_routes(oracle.gemv_ref, oracle.gemv_ref_real)


def test_gemv_converges_to_real_layer():
    pins.check_gemv_lossless(oracle.gemv_ref, oracle.quantize, oracle.split)
