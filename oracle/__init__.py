"""CPU fp64 oracle of the dropless MoE expert layer.

TEST INFRASTRUCTURE ONLY. It is imported by the tests, by the smoke check and
by the benchmark's CPU-baseline leg, and by nothing else. It shares no code
with the HIP library: it is a plain, slow, per-expert implementation written
from the pages, used to prove the GPU path right.
"""
from .moe_oracle import (  # noqa: F401
    router_logits, selection_keys, topk_select, gate_weights, route,
    permute, swiglu, expert_ffn, forward, forward_gather, dense_masked_forward,
    stage_gemm1, stage_gemm2, stage_combine, backward, backward_sampled,
    gate_logit_grad, router_backward, gate_probs, load_balance_stats,
    aux_loss_logit_grad, update_route_bias, balance_monitor,
)
from .mxfp8 import (  # noqa: F401
    e4m3_values, e4m3_round, mx_quantize, mx_dequantize, mx_roundtrip,
    forward_mxfp8, mx_roundtrip_cols, backward_mxfp8, backward_mxfp8_sampled,
)
