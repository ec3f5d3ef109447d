"""Oracle pins: per-token int8 activations, integer plane GEMM and its epilogue."""
import oracle
import pins


def test_act_quant_golden():
    pins.check_act_quant_golden(oracle.act_quant_ref)


def test_act_quant_properties():
    pins.check_act_quant_props(oracle.act_quant_ref)


def test_gemm_int_two_routes():
    pins.check_gemm_routes(oracle.gemm_int_ref, oracle.gemm_int_ref_loops)


def test_gemm_epilogue_is_gemv_of_dequantized_activations():
    pins.check_gemm_epilogue(oracle.gemm_int_ref, oracle.gemm_epilogue_ref, oracle.gemv_ref)
