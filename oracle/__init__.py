"""CPU oracle (float64) for projection -> residual add -> RMSNorm.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library.
"""
from .reference import (E4M3_MAX, NORM_GEMMA, NORM_STANDARD, OUT_MAX_ABS, OUT_REL_L2,
                        RES_REL_L2, bf16_bits_of, compare, conventional_roundings, decode_e4m3,
                        encode_e4m3, norm_gain, proj_add_rmsnorm, proj_add_rmsnorm_chunked,
                        proj_add_rmsnorm_conventional_taken, proj_add_rmsnorm_fp8,
                        projection, projection_fp8, quantize_fp8, residual_add, rms_norm,
                        round_bf16, silu_mul, widen_bf16, widen_f32, within_tolerance)

__all__ = [
    "E4M3_MAX", "decode_e4m3", "encode_e4m3", "proj_add_rmsnorm_fp8", "projection_fp8",
    "quantize_fp8", "NORM_GEMMA", "NORM_STANDARD", "OUT_MAX_ABS", "OUT_REL_L2", "RES_REL_L2", "bf16_bits_of",
    "compare", "conventional_roundings", "norm_gain", "proj_add_rmsnorm",
    "proj_add_rmsnorm_chunked", "proj_add_rmsnorm_conventional_taken", "projection",
    "residual_add", "rms_norm", "round_bf16", "silu_mul", "widen_bf16", "widen_f32",
    "within_tolerance",
]
