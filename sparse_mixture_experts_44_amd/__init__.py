"""Forward (and backward) pass of a top-k routed Mixture-of-Experts layer on AMD MI355X (gfx950).

libmoe.so holds the hand-written HIP kernels behind a C ABI (include/moe.h).
This package is its ctypes binding, with the same names, plus MoELayer, which
keeps the weights resident on the device. Importing the package does not load
the library; the first call does, and fails loudly if it has not been built.
"""
from ._native import (  # noqa: F401
    LIB_PATH, MOE_DTYPE_BF16, MOE_DTYPE_F32, MOE_ERR_HIP, MOE_GRAD_ACCUMULATE, MOE_GRAD_WRITE, MOE_GRAD_WRITE_BF16, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE, MOE_OK, MOE_STAGE_EVENTS, STAGES, MoEError, MoEFp8Scales, MoEShape,
    MoEWeightScales, backward_workspace_bytes, fp8_scales, lib, moe_backward, moe_combine, moe_forward,
    MOE_NOALLOC_SCRATCH_BYTES, moe_forward_fp8, moe_forward_int4, moe_forward_noalloc, moe_forward_train, moe_grouped_swiglu, moe_grouped_swiglu_fp8,
    moe_grouped_swiglu_int4, moe_permute, moe_dequantize_fp8, moe_quantize_fp8, moe_quantize_int4, moe_route, moe_router_aux,
    moe_update_select_bias, status_string, train_save_floats, weight_scales, workspace_bytes,
)


def shape_for(cfg, n_tokens=None) -> MoEShape:
    """MoEShape of a moe_inputs.MoEConfig."""
    return MoEShape.make(cfg.n_tokens if n_tokens is None else n_tokens, cfg.d_model, cfg.d_ff,
                         cfg.n_experts, cfg.top_k, cfg.n_shared, cfg.d_ff_shared, cfg.capacity,
                         cfg.renormalize, MOE_DTYPE_BF16 if cfg.dtype == "bf16" else MOE_DTYPE_F32)
