"""DeepSeekMoE feed-forward layer on one MI355X (gfx950): HIP kernels behind a
C ABI (include/dsmoe.h), with this thin Python binding on top."""
from ._lib import (MOE_DT_BF16, MOE_DT_F32, MOE_DT_FP8_E4M3, MoeError, MoeLayerDesc, MoeWeights,
                   deepseek_moe_forward, deepseek_moe_forward_noalloc, lib, make_weights, moe_abi_version, moe_bias_update,
                   moe_combine, moe_expert_ffn, moe_gate, moe_permute, moe_profile_events, moe_quantize_fp8_blocks,
                   moe_quantize_fp8_rows, moe_route_from_logits, moe_workspace_size,
                   moe_backward, moe_backward_workspace_size, moe_forward_train,
                   moe_seq_balance_loss, moe_seq_balance_workspace_size,
                   moe_backward_fp8, moe_transpose_fp8_blocks)
from .layer import MoELayer, make_desc, quantize_fp8_blocks
from .workloads import CONFIGS, Workload, make_inputs, make_layer, make_tokens

__all__ = [
    "MOE_DT_BF16", "MOE_DT_F32", "MOE_DT_FP8_E4M3", "MoeError", "MoeLayerDesc", "MoeWeights",
    "deepseek_moe_forward", "deepseek_moe_forward_noalloc", "lib", "make_weights", "moe_abi_version", "moe_bias_update",
    "moe_combine", "moe_expert_ffn", "moe_gate", "moe_permute", "moe_profile_events", "moe_quantize_fp8_blocks",
    "moe_quantize_fp8_rows", "moe_route_from_logits", "moe_workspace_size", "MoELayer",
    "make_desc", "quantize_fp8_blocks", "CONFIGS", "Workload", "make_inputs", "make_layer",
    "make_tokens", "moe_backward", "moe_backward_workspace_size", "moe_forward_train",
    "moe_seq_balance_loss", "moe_seq_balance_workspace_size", "moe_backward_fp8",
    "moe_transpose_fp8_blocks",
]
