"""CPU oracle for the AQLM quantized linear layer (test infrastructure only).

Only the test suite, the smoke entry point and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its binding)
never calls it and shares no code with it.
"""
from .aqlm_oracle import (  # noqa: F401
    SUPPORTED_SCHEMES,
    codes_to_index,
    decode_fp32,
    decode_fp16,
    decode_loop,
    linear_ref_f64,
    linear_ref_rows_f64,
    bits_per_weight,
    bits_per_weight_terms,
    parity_errors,
    within_tolerance,
    pack_codes,
    unpack_codes,
    packed_words,
    packed_to_stored,
    decode_fp32_packed,
)
