"""CPU oracle for the Fairy2i widely-linear 2-bit path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct float64 / int64 NumPy code that states what the
GPU library must compute.  Only the test suite, the smoke check in
`__graft_entry__` and the CPU-baseline leg of `bench.py` may import it; the
product path (`widely_linear_gemv_amd`) never does, and the oracle never
imports the product path.  The two share no code: the only common input is the
seeded generator module `workloads`, which holds none of the method's
arithmetic.

Sources (the pages, cited by title and section):
  * ModelScope model card "Fairy2i-W2", section "Method" (widely-linear
    transform; phase-aware complex quantization; recursive residual
    quantization) and "Model details".
  * zhichai.net reading note "Fairy2i: Ultra-Low-Bit LLM Quantization Using
    Complex Weights {+-1, +-i}": "Step 1" (Theorem 1 and the block closed
    form), "Step 2" (projection and dequantization), "Step 3" (residual
    recursion), "Industry implications: multiplication-free inference".
  * 36Kr article "The 2-bit complex model rivals full precision ...",
    points 1-3 and the multiplication-free / parallel-stage paragraphs.

Where the pages leave a step open the oracle takes one reading and says so in
the function's docstring.  Every function here is pinned by the `-m "not gpu"`
tests against facts that do not come from the oracle itself (closed forms,
brute force, identities, hand-worked fixtures under tests/golden/).
Model quality (perplexity, zero-shot accuracy) needs trained weights and
datasets and is parity unpinned; nothing here computes it.
"""
from .widely_linear import split, unsplit
from .phase_quant import project, ordered_row_sum, quantize, dequantize, dequantize_real, REDUCE_LANES
from .packing import pack, pack_words, unpack, packed_nbytes
from .gemv import gemv_ref, gemv_ref_real, code_planes
from .prefill import act_quant_ref, gemm_int_ref, gemm_int_ref_loops, gemm_epilogue_ref

__all__ = [
    "split", "unsplit", "project", "ordered_row_sum", "quantize", "dequantize", "dequantize_real", "REDUCE_LANES",
    "pack", "pack_words", "unpack", "packed_nbytes", "gemv_ref", "gemv_ref_real", "code_planes",
    "act_quant_ref", "gemm_int_ref", "gemm_int_ref_loops", "gemm_epilogue_ref",
]
