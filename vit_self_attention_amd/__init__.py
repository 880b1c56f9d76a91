"""libvitattn: the vision-encoder self-attention forward on MI355X (gfx950).

    import vit_self_attention_amd as va
    out = va.fwd(qkv)            # qkv: bf16 or fp16 [B, N, 3, H, D] -> out [B, N, H, D]
    out = va.fwd(q, k, v)        # q, k, v: bf16 [B, H, N, D] -> out [B, H, N, D]
    qkv = va.linear(x, w_qkv, b_qkv)            # the block's qkv projection: [B, N, 3*H*D]
    y = va.linear(o, w_proj, b_proj, residual=x) # output projection + bias + residual
    plan = va.Plan(qkv_per_layer) # the same calls recorded once into a HIP graph
    plan.launch()

The computation runs in the HIP kernels of libvitattn.so through its C ABI
(include/vitattn.h); this package only marshals arguments.
"""
from ._binding import (ERR_BAD_LAYOUT, ERR_BAD_SCALE, ERR_BAD_SIZE, ERR_GRAPH, ERR_LAUNCH,
                       ERR_MISALIGNED, ERR_NULL_POINTER, ERR_OVERLAP, ERR_TOO_LARGE,
                       ERR_UNSUPPORTED_D, ERR_UNSUPPORTED_SHAPE, EXPORTED, DTYPE_FP16,
                       LAYOUT_PACKED, LAYOUT_SEPARATE, LIBRARY, OK, Plan, VitAttnError, fwd,
                       fwd_args, fwd_c, fwd_raw, fwd_shape, linear, linear_raw, plan_create_raw, plan_destroy_raw,
                       plan_launch_raw, strerror, version)

__all__ = ["fwd", "fwd_args", "fwd_c", "fwd_raw", "fwd_shape", "linear", "linear_raw", "Plan", "plan_create_raw", "plan_launch_raw", "plan_destroy_raw",
           "strerror", "version", "VitAttnError", "LAYOUT_PACKED", "LAYOUT_SEPARATE", "DTYPE_FP16",
           "LIBRARY",
           "EXPORTED"]
