"""int4 routed-expert MoE layer on AMD Instinct MI355X (gfx950).

The compute lives in ``libmoe_int4.so`` (hand-written HIP kernels behind the
C ABI in ``include/moe_int4.h``); this package is its ctypes binding plus
helpers that allocate the caller-owned device buffers with PyTorch.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_BF16, MOE_F32, MOE_OK, MOE_PATH_DECODE_F32, MOE_PATH_PREFILL_BF16,
    MOE_QUANT_GS64, MOE_QUANT_ROW, MoeError, Shape, STATUS_NAMES, load, moe_combine,
    moe_expert_bytes, moe_expert_ffn, moe_ffn_workspace_bytes, moe_layer_decode,
    moe_layer_decode_workspace_bytes, moe_layer_decode_static, moe_layer_decode_static_max_bytes,
    moe_pack_experts, moe_quantize,
    moe_route, moe_route_union, moe_route_workspace_bytes, moe_status_str, moe_union,
    moe_cache_create, moe_cache_destroy, moe_cache_layer_decode, moe_cache_pin, moe_cache_plan,
    moe_cache_stats, moe_cache_last_fetch, moe_cache_unplan_last, moe_cache_workspace_bytes, moe_measure_stream_read,
)


def shape_of(layer_shape) -> Shape:
    """moe_shape of a synthetic layer description (anything with d, f,
    n_experts, top_k, f_shared and group attributes)."""
    return Shape(layer_shape.d, layer_shape.f, layer_shape.n_experts, layer_shape.top_k,
                 getattr(layer_shape, "group", 64), layer_shape.f_shared)
