"""CPU oracle (float64) for projection -> residual add -> RMSNorm.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library.
"""
from .reference import (NORM_GEMMA, NORM_STANDARD, OUT_MAX_ABS, OUT_REL_L2, RES_REL_L2,
                        bf16_bits_of, compare, norm_gain, proj_add_rmsnorm,
                        proj_add_rmsnorm_chunked, projection, residual_add, rms_norm,
                        round_bf16, silu_mul, widen_bf16, widen_f32, within_tolerance)

__all__ = [
    "NORM_GEMMA", "NORM_STANDARD", "OUT_MAX_ABS", "OUT_REL_L2", "RES_REL_L2", "bf16_bits_of",
    "compare", "norm_gain", "proj_add_rmsnorm", "proj_add_rmsnorm_chunked", "projection",
    "residual_add", "rms_norm", "round_bf16", "silu_mul", "widen_bf16", "widen_f32",
    "within_tolerance",
]
