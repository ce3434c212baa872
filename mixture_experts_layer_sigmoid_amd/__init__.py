"""Sigmoid-routed MoE layer for AMD Instinct MI355X (gfx950).

The layer (router with selection-only bias and grouped top-k, expert-major
permute, grouped fc1 + SwiGLU, grouped fc2, weighted combine, MX
and NVFP4 quantization) runs in the hand-written HIP library libmoe_mi355x.so behind
the C ABI of include/moe_mi355x.h. This package is its Python binding: the
functions in `_lib` carry the C names and only marshal arguments; `layer`
strings them into a forward pass. There is no CPU fallback: every binding call
loads the built library and raises when it is missing.
"""
from ._lib import (  # noqa: F401
    load, MoEError, MOE_F32, MOE_BF16, MOE_MXFP8_E4M3, MOE_MXFP4_E2M1, MOE_NVFP4_E2M1,
    moe_abi_version, moe_route, moe_route_workspace, moe_quantize_mx, moe_permute_rows_bound,
    moe_permute_workspace, moe_permute, moe_permute_noalloc, moe_permute_noalloc_max_bytes,
    moe_grouped_mlp_workspace,
    moe_grouped_mlp_fwd, moe_grouped_fc1_swiglu, moe_grouped_fc2, moe_combine,
    moe_grouped_fc1_swiglu_dense, moe_grouped_fc2_dense,
    moe_pack_weights, moe_combine_bwd, moe_unpermute, moe_segments_kstride, moe_quantize_mx_segments,
    moe_grouped_fc2_dgrad_dswiglu, moe_grouped_fc1_dgrad, moe_grouped_wgrad,
    moe_grouped_mlp_bwd, moe_grouped_mlp_bwd_workspace, moe_route_bwd, moe_route_bwd_workspace,
    moe_bias_update, moe_nvfp4_tensor_scale, moe_quantize_nvfp4, moe_grouped_fc1_swiglu_nvfp4,
    moe_grouped_fc2_nvfp4,
    SIGNATURES, LIB_PATH,
)
from .layer import (MoEForward, MoEBackward, RouterBackward, ExpertWeights, bias_update,  # noqa: F401
                    quantize_mx, quantize_mx_t, FMT)
