"""CPU fp64 oracle for the exact-attention forward and its FP8 variant.

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark -- never by the HIP path, which shares
no code with it (only the seeded input generator serves both).
"""
from .attention import (attention, attention_backward, attention_backward_head, attention_backward_rows,
                        attention_head, attention_partial, attention_rows, credited_flops, merge_partials, row_softmax,
                        scores)
from .fp8 import (E4M3_MAX, E5M2_MAX, FORMATS, attention_fp8_simulated, block_quantize, dequantize,
                  e4m3_decode, e4m3_encode, e5m2_decode, e5m2_encode, hadamard_rotate_quant, quantized_probabilities, rel_rms, rotate,
                  sylvester_hadamard)
from .rope import rope, rope_angles, rope_hadamard_rotate_quant

__all__ = [
    "attention", "attention_backward", "attention_backward_head", "attention_backward_rows", "attention_head", "attention_partial", "attention_rows", "credited_flops",
    "merge_partials", "row_softmax",
    "scores", "E4M3_MAX", "E5M2_MAX", "FORMATS", "attention_fp8_simulated", "block_quantize",
    "dequantize", "e4m3_decode", "e4m3_encode", "e5m2_decode", "e5m2_encode", "hadamard_rotate_quant", "quantized_probabilities", "rel_rms", "rotate",
    "sylvester_hadamard", "rope", "rope_angles", "rope_hadamard_rotate_quant",
]
