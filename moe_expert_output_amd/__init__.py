"""MI355X (gfx950) MoE finalize: gather the top-k permuted expert rows, float32 weighted sum,
routed scaling, shared-expert add, one rounding, residual add, RMSNorm, optional FP8 / NVFP4.

The compute lives in libmoe_finalize.so (hand-written HIP, C ABI in include/moe_finalize.h);
`binding` is a ctypes layer with the same entry-point names.
"""
from .binding import (  # noqa: F401
    EXPORTED, LAUNCH_CONFIG_FIELDS, LIB, MOE_DTYPE_BF16, MOE_DTYPE_FP16, MOE_DTYPE_FP32,
    MOE_FIN_CACHE_AUTO, MOE_FIN_CACHE_KEEP, MOE_FIN_CACHE_STREAM, MOE_QUANT_FP8_E4M3,
    MOE_QUANT_NVFP4, MOE_SF_LINEAR, MOE_SF_SWIZZLED_128x4, MoeFinalizeError,
    moe_finalize_error_string, moe_finalize_launch_config, moe_finalize_launch_floor_run,
    moe_finalize_quant_run, moe_finalize_rmsnorm_noalloc_run, moe_finalize_rmsnorm_run,
    moe_finalize_run,
    moe_finalize_set_cache_policy, moe_finalize_set_wait_limit, moe_finalize_sf_size,
    moe_finalize_stream_floor_run, moe_finalize_stream_probe_run, moe_finalize_version,
    moe_finalize_workspace_flag, moe_finalize_workspace_size,
    moe_quantize_run, moe_rank_sum_quant_run, moe_rank_sum_rmsnorm_run, moe_residual_rmsnorm_run,
)
