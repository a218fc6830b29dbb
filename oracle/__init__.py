"""CPU oracle (test infrastructure only; see ``w4_oracle``)."""

from .w4_oracle import (  # noqa: F401
    GROUP, QMAX, f32, ieee_div, round_away, clamp_code, to_code, fp16_bits, fp16_value,
    quantize_group_scalar, quantize_scalar, dot_scalar, dot_factored_exact,
    quantize_ref, unpack_codes, dequant_ref, gemv_ref, gemv_factored_ref,
    tolerance_ref, bits_per_weight, quantize_symmetric_ref, SYM_ZERO,
    quantize_ref_f32, quantize_symmetric_ref_f32,
)
from .w4_formats import (  # noqa: F401
    Format, CANONICAL, bf16_bits, bf16_value, scale_value, pack_zero_nibbles,
    unpack_zero_nibbles, zero_bytes, quantize_format_ref, zeros_u8, dequant_format_ref,
    gemv_format_ref, tolerance_format_ref, format_bits_per_weight, format_bytes,
)
from .fp8_oracle import (  # noqa: F401
    FP8_MAX, E4M3_VALUES, e4m3_decode, e4m3_encode, quantize_rows_fp8_ref, dequant_fp8_ref,
    gemm_fp8_ref, tolerance_fp8_ref,
)
from .int8_oracle import (  # noqa: F401
    INT8_MAX, quantize_rows_int8_ref, dequant_int8_ref, gemm_int8_ref, tolerance_int8_ref,
)
