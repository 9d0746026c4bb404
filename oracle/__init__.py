"""CPU oracle for the FP8 scaled matrix multiply.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library and its Python binding never
import it.
"""
from .fp8_scaled_mm_ref import (  # noqa: F401
    PER_TENSOR, ROWWISE, E4M3FN, E5M2, FORMAT_NAMES, UNIT_EXP, e4m3fn_value, e5m2_value,
    e4m3fn_decode_table, e5m2_decode_table, decode, bf16_bits_to_f64, f64_to_bf16_rne,
    scaled_mm,
)
from .quantize_ref import (  # noqa: F401,E402
    E4M3_MAX, E5M2_MAX, FORMATS, encode_rne, e4m3fn_encode_rne, quantize, quantize_e4m3,
    dequantize,
)
