"""MI355X-native (gfx950) int4/int8 group-quantized sparse MoE layer.

The compute path is the HIP library ``libmoe.so`` built from ``csrc/``; this
package is its ctypes binding (same entry-point names as include/moe.h) plus
a small descriptor helper.  PyTorch is used only for device memory and
streams.
"""
from ._ffi import (  # noqa: F401
    MOE_ACT_BF16, MOE_ACT_F32, MOE_ERR_INVALID_ARG, MOE_ERR_LAUNCH, MOE_ERR_MISALIGNED,
    MOE_ERR_NO_DEVICE, MOE_ERR_TOO_LARGE, MOE_ERR_UNSUPPORTED, MOE_FLAG_ROUTER_BIAS,
    MOE_FLAG_SHARED, MOE_FLAG_DENSE_Q4, MOE_NOALLOC_SCRATCH_BYTES, MOE_OK,
    MoeError, exported_symbols, lib, moe_blob_layout, moe_blob_layout_t, moe_chain_forward,
    moe_chain_status, moe_experts_forward, moe_layer_desc, moe_layer_forward,
    moe_layer_forward_noalloc, moe_pack_expert, moe_dense_layout, moe_dense_layout_t,
    moe_pack_dense,
    moe_pack_experts_device, moe_residual_rmsnorm, moe_rmsnorm, moe_router_topk,
    moe_status_string, moe_version, moe_workspace_bytes, moe_workspace_routing,
    moe_gdn_desc, moe_attn_desc, make_gdn_desc, make_attn_desc, moe_gdn_decode,
    moe_attn_workspace_bytes, moe_attn_decode, MoePool, MOE_POOL_HOST_ONLY,
)


def make_desc(n_tokens, hidden, n_experts, top_k, inter, shared_inter=0, bits=4, act="bf16",
              expert_stride=0, router_bias=False, shared=True, rms_eps=1e-6, group=64,
              dense_q4=False):
    """Build a moe_layer_desc; expert_stride=0 means the blob size."""
    d = moe_layer_desc()
    d.n_tokens, d.hidden, d.n_experts, d.top_k = n_tokens, hidden, n_experts, top_k
    d.inter, d.shared_inter, d.group, d.bits = inter, shared_inter if shared else 0, group, bits
    d.act_dtype = MOE_ACT_BF16 if act == "bf16" else MOE_ACT_F32
    d.flags = ((MOE_FLAG_ROUTER_BIAS if router_bias else 0) | (MOE_FLAG_SHARED if shared else 0)
               | (MOE_FLAG_DENSE_Q4 if dense_q4 else 0))
    d.rms_eps = rms_eps
    if expert_stride == 0:
        d.expert_stride = 0
        expert_stride = moe_blob_layout(d, inter).blob_bytes
    d.expert_stride = expert_stride
    return d
