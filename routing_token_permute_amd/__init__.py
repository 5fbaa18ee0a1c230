"""MI355X-native single-GPU MoE expert layer: forward and backward.

The layer (router, softmax/top-K, expert-major permutation with counts,
offsets and splits, grouped SwiGLU GEMM, weighted combine) and its gradient
run in the HIP kernels of libmoe.so behind the C ABI in include/moe.h; this
package is its Python binding. Build the library with `python -m routing_token_permute_amd.build`.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MOE_BF16,
    MOE_F32,
    MoEError,
    device_info,
    load_library,
    moe_backward,
    moe_backward_workspace_size,
    moe_combine_backward,
    moe_dispatch_backward,
    moe_expert_w2,
    moe_expert_w2_backward,
    moe_expert_w2_fp8,
    moe_expert_w2_scatter,
    moe_expert_w13_swiglu,
    moe_expert_w13_backward,
    moe_expert_w13_swiglu_gather,
    moe_expert_w13_swiglu_gather_fp8,
    moe_expert_w13_swiglu_gather_train,
    moe_expert_weight_grad,
    moe_expert_weight_grad_gather,
    moe_forward,
    moe_forward_fp8,
    moe_forward_noalloc,
    moe_forward_train,
    moe_forward_workspace_size,
    moe_grouped_swiglu,
    moe_permute,
    moe_quantize_fp8,
    moe_route,
    moe_route_backward,
    moe_sum_slots,
    moe_unpermute_combine,
    status_string,
)
