"""MI355X-native sparse MoE layer (route, permute, expert-slot cache, FP4 expert FFN, combine).

The product is the C-ABI library ``libmoe.so`` (HIP kernels for gfx950, see
``include/moe.h``); ``fp4_expert_ffn_amd._lib`` is its ctypes binding with the
same names, and ``fp4_expert_ffn_amd.layer`` chains the calls for one layer.
"""
from ._lib import (  # noqa: F401
    AMODE, FMT, BwCalib, LayerArgs, Cache, CachePrefill, CacheStep, Hybrid, FfnArgs, MoeError, cache_fill, cache_lookup, ffn_args, lib, moe_blob_bytes,
    moe_cache_create, moe_cache_decode_step, moe_cache_decode_step_hybrid, moe_calibrate_bw, moe_cpu_expert_ffn, moe_cache_destroy, moe_cache_map_bytes, moe_cache_mark_used,
    moe_cache_pin_resident, moe_cache_prefetch_layer, moe_cache_prefill_step, moe_cache_reset, moe_cache_resize, moe_cache_stats, moe_cache_use_copy_engine, moe_combine, moe_debug_fp4_codes, moe_dequant_blob, moe_expert_ffn, moe_expert_ffn_noalloc,
    moe_expert_ffn_traced, moe_expert_ffn_workspace_size, moe_last_error, moe_layer, moe_layer_traced, moe_permute, moe_prepack_expert, moe_quantize_mxfp4, moe_route,
    moe_route_permute, moe_router_logits, moe_version,
)
