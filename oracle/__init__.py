"""CPU float64 oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition that the GPU path is checked against. Only the test-suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does.
"""
from .attention import (  # noqa: F401
    scores,
    probabilities,
    forward,
    forward_quantized,
    backward,
    backward_rows,
    backward_causal_tail,
    forward_gqa,
    backward_gqa,
    forward_decode,
    backward_quantized,
    softmax_by_chunks,
    brute_force_forward,
    brute_force_backward,
    decode_e4m3fn,
    decode_e5m2,
)
