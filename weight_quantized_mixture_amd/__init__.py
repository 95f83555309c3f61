"""Weight-only-quantized fused MoE layer for MI355X (gfx950).

The compute lives in the HIP library ``libmoe_wq.so`` (C ABI: include/moe_wq.h);
``binding`` marshals torch tensors into its calls and ``layer`` holds the
parameters the way the experts_int8 and moe_wna16 pages name them.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MOE_BF16,
    MOE_FP16,
    lib,
    moe_align_block,
    moe_align_capacity,
    moe_combine_topk,
    moe_quantize_weights_int8,
    moe_quantize_weights_w4,
    moe_route_select,
    moe_route_topk,
    moe_fp8_merge_w13_scales,
    moe_quantize_weights_fp8,
    moe_wfp8a16_apply,
    moe_wfp8a16_forward,
    moe_wfp8a16_workspace_bytes,
    moe_quantize_act_int8,
    moe_w8a8_apply,
    moe_w8a8_forward,
    moe_w8a8_workspace_bytes,
    moe_w4_import,
    moe_wna16_group_size,
    moe_w4a16_apply,
    moe_w4a16_apply_ex,
    moe_w4a16_forward_ex,
    moe_w4a16_workspace_bytes_ex,
    moe_w8a16_apply_ex,
    moe_w8a16_forward_ex,
    moe_w8a16_workspace_bytes_ex,
    moe_w4a16_forward,
    moe_w4a16_workspace_bytes,
    moe_w8a16_apply,
    moe_w8a16_block_m,
    moe_w8a16_forward,
    moe_w8a16_gemm1,
    moe_w8a16_gemm2,
    moe_w8a16_splits,
    moe_w8a16_intermediate_bytes,
    moe_w8a16_requant,
    moe_w8a16_workspace_bytes,
)
from .layer import W4A16MoE, W8A16MoE, WFP8A16MoE  # noqa: F401
