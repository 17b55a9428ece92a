"""MI355X-native DeepSeekMoE layer forward: HIP kernels for gfx950 behind a C ABI.

The kernels and the C ABI live in ``csrc/`` and build into ``libmoe.so``
(``python -m sparse_moe_layer_affinity_amd.build``); ``binding`` exposes the same
entry points to Python.  Importing this package does not load the library.
"""
from .binding import (MoeConfig, MoeError, MoeExpertWeights, lib, make_config,  # noqa: F401
                      moe_act_quant_e4m3, moe_balance_loss, moe_bias_update, moe_combine,
                      moe_combine_backward, moe_gate_backward, moe_grouped_ffn, moe_router_scores,
                      moe_swiglu_backward, moe_backward_workspace_bytes,
                      moe_expert_backward_input, moe_expert_backward, moe_router_backward,
                      moe_router_backward_workspace_bytes,
                      moe_layer_forward, moe_layer_forward_noalloc, moe_permute, moe_route,
                      moe_status_string,
                      moe_workspace_bytes, DTYPE_CODES)
