"""Algorithmic FLOP and byte counts of the MoE layer (what the method must
do: no padding, no dense all-expert work).

Sources: quant67.com, "【大模型基础设施工程】08：MoE 训练工程", §9 (a SwiGLU
expert is three d_model x d_ff linear layers), §14.5.1 (training compute is
about 6 x active parameters x tokens, i.e. forward plus a backward of twice
the forward) and §14.5.3 (token-copy traffic per layer is about
2 x K x D x bytes per token: one copy out to the experts, one back).
"""
from __future__ import annotations


def gemm1_flops(d: int, f: int, copies: int) -> int:
    """x W1^T and x W3^T over every routed copy: 2 GEMMs x 2 flops/MAC."""
    return 4 * d * f * copies


def gemm2_flops(d: int, f: int, copies: int) -> int:
    """h W2^T over every routed copy."""
    return 2 * d * f * copies


def routed_fwd_flops(d: int, f: int, copies: int) -> int:
    """Three d x f GEMMs per routed copy (SwiGLU elementwise work is not
    counted)."""
    return 6 * d * f * copies


def shared_fwd_flops(d: int, f_shared: int, T: int) -> int:
    return 6 * d * f_shared * T


def router_flops(T: int, d: int, E: int) -> int:
    return 2 * T * d * E


def train_flops(fwd_flops: float) -> float:
    """Forward plus backward: backward costs two forwards (dgrad + wgrad)."""
    return 3 * fwd_flops


def training_flops_6nt(n_active: float, tokens: float) -> float:
    """The pages' training-compute estimate, 6 x N_act x T."""
    return 6.0 * n_active * tokens


def comm_bytes_per_token(K: int, D: int, bytes_per_elem: int) -> int:
    """Token-copy traffic per token and layer: K copies out, K back."""
    return 2 * K * D * bytes_per_elem


def permute_bytes(T: int, K: int, d: int, b: int) -> int:
    """Read x once, write T*K rows of x_perm; read topk_idx and write
    sorted_src and dest (three int32 per copy)."""
    return T * d * b + T * K * d * b + 12 * T * K


def permute_index_bytes(T: int, K: int) -> int:
    """The permute when GEMM 1 gathers its rows: read topk_idx, write
    sorted_src and dest (three int32 per copy), no rows."""
    return 12 * T * K


def quantize_bytes(n: int) -> float:
    """MX quantisation of n bf16 elements: read 2n, write n codes and n/32
    scales."""
    return 2 * n + n + n / 32


def combine_bytes(T: int, K: int, d: int, b: int, shared: bool) -> int:
    """Read T*K rows of y_perm, (read y_shared,) write out; read dest and
    topk_w (int32 + fp32 per copy)."""
    return T * K * d * b + T * d * b * (2 if shared else 1) + 8 * T * K


def expert_weight_bytes(E: int, d: int, f: int, b: int) -> int:
    return 3 * E * d * f * b


def gemm1_bytes(E: int, d: int, f: int, copies: int, b: float) -> float:
    """Grouped GEMM 1 + SwiGLU: read x_perm and W1, W3 once, write h.
    For MXFP8 pass b = 1 + 1/32 (one E8M0 scale per 32 elements)."""
    return copies * d * b + 2 * E * f * d * b + copies * f * b
