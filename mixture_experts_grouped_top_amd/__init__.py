"""MoE expert-FFN path for MI355X (gfx950): HIP kernels behind a C ABI.

The shared library ``libmoe.so`` (built from ``csrc/`` by
``python -m mixture_experts_grouped_top_amd.build``) exports the entry
points declared in ``include/moe.h``.  This package binds them by name
(argument marshalling only) and sequences them into a forward/backward
plan.  Importing the package does not load the library; the first call
does, and raises if it has not been built.
"""
from ._binding import (MOE_BF16, MOE_BIAS_LOGIT, MOE_BIAS_SELECT, MOE_DERR_EXPERT_ID,
                       MOE_DERR_GROUP_SIZES, MOE_DERR_ROWS, MOE_F32, MOE_SIGMOID, MOE_SOFTMAX,
                       SIGNATURES, MoeError, load, moe_aux_loss, moe_aux_loss_bwd,
                       moe_aux_loss_workspace, moe_combine, moe_combine_bwd, moe_gmm, moe_gmm_swiglu,
                       moe_gmm_swiglu_bwd,
                       moe_group_sum, moe_group_sum_workspace, moe_router_bwd,
                       moe_router_bwd_workspace, ABI_VERSION,
                       MOE_FP8_E4M3, MOE_FP8_E5M2, moe_fp8_scale_workspace, moe_fp8_amax_scale,
                       moe_fp8_padded_rows, moe_fp8_quantize, moe_gmm_fp8, moe_tgmm_fp8,
                       moe_permute, moe_permute_bwd, moe_permute_workspace, moe_route,
                       moe_route_bwd, moe_rows_bound, moe_swiglu, moe_swiglu_bwd, moe_tgmm,
                       LIB_PATH)
from .block import MoEPlan, MoEShape

__all__ = [
    "load", "MoeError", "LIB_PATH", "SIGNATURES", "moe_route", "moe_route_bwd", "moe_rows_bound",
    "moe_aux_loss_workspace", "moe_aux_loss", "moe_aux_loss_bwd", "MOE_BIAS_LOGIT",
    "MOE_BIAS_SELECT",
    "moe_permute_workspace", "moe_permute", "moe_permute_bwd", "moe_gmm", "moe_gmm_swiglu", "moe_gmm_swiglu_bwd", "moe_tgmm",
    "moe_group_sum_workspace", "moe_group_sum", "moe_router_bwd", "moe_router_bwd_workspace",
    "ABI_VERSION", "MOE_FP8_E4M3", "MOE_FP8_E5M2",
    "moe_fp8_scale_workspace", "moe_fp8_amax_scale", "moe_fp8_padded_rows", "moe_fp8_quantize",
    "moe_gmm_fp8", "moe_tgmm_fp8",
    "moe_swiglu", "moe_swiglu_bwd", "moe_combine", "moe_combine_bwd", "MoEPlan", "MoEShape",
    "MOE_F32", "MOE_BF16", "MOE_SOFTMAX", "MOE_SIGMOID", "MOE_DERR_EXPERT_ID",
    "MOE_DERR_GROUP_SIZES", "MOE_DERR_ROWS",
]
