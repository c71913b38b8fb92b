"""MI355X-native forward pass of one Mixture-of-Experts layer.

gate (float32 logits, top-k, renormalised weights) -> dispatch (histogram,
scan, stable permutation, optional per-token affine FP8 rows) -> grouped
SwiGLU expert FFN (bf16 matrix cores) -> combine (weighted un-permute).
The work runs in the HIP kernels of libmoe_mi355x.so behind the C ABI in
include/moe.h; this package is its ctypes binding. Build the library with
``python mixture_experts_routing_gemm_amd/build.py``.
"""

from ._binding import (  # noqa: F401
    EXPORTS, MOE_BF16, MOE_ERR_BAD_INDEX, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE, MOE_F32, MOE_FP8_E4M3, MOE_OK, MOE_OVERFLOW_DROP, MOE_OVERFLOW_REASSIGN,
    MOE_QUANT_EXPERT, MOE_QUANT_GLOBAL, MOE_QUANT_TOKEN, MOE_QUANT_TOKEN_ABSMAX,
    FP8W_KERNELS, STAGE_COMBINE, STAGE_DISPATCH, STAGE_FFN, STAGE_FFN_BACKWARD, STAGE_FORWARD_FP8W,
    STAGE_GATE_BACKWARD,
    STAGE_FORWARD, STAGE_GATE, MoEError, alloc_workspace, make_shape, moe_combine, moe_combine_backward,
    moe_dispatch, moe_dispatch_backward, moe_dispatch_noalloc, moe_gate_backward,
    moe_forward, moe_forward_fp8w, moe_forward_kernel_count, moe_fp8_weight_scale_floats,
    moe_quantize_weights, moe_forward_kernel_name, moe_forward_traced,
    moe_gate_topk, moe_get_device_error, moe_grouped_ffn, moe_grouped_ffn_backward, moe_shape,
    moe_ffn_saved_bytes, alloc_saved, moe_grouped_ffn_save, moe_grouped_ffn_backward_saved,
    moe_workspace_bytes,
    moe_workspace_init, shape_of, status_string)
from .buffers import ForwardBuffers  # noqa: F401
