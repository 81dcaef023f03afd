"""Buffer allocation and argument packing for whole-layer calls.

Allocation is done with torch (device memory is torch's); the packed
argument structs are handed to moe_forward / moe_backward unchanged.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import binding as B


def act_torch_dtype(desc: B.MoeDesc) -> torch.dtype:
    return torch.float32 if desc.act_dtype == B.MOE_F32 else torch.bfloat16


def alloc_forward(desc: B.MoeDesc, device="cuda") -> dict:
    """Every caller-owned forward buffer for ``desc`` plus the workspace."""
    T, d, f, E, K = desc.T, desc.d_model, desc.d_ff, desc.E, desc.K
    TK = T * K
    dt = act_torch_dtype(desc)
    i32 = torch.int32
    bufs = {
        "out": torch.empty(T, d, dtype=dt, device=device),
        "logits": torch.empty(T, E, dtype=torch.float32, device=device),
        "topk_idx": torch.empty(T, K, dtype=i32, device=device),
        "topk_w": torch.empty(T, K, dtype=torch.float32, device=device),
        "counts": torch.empty(E, dtype=i32, device=device),
        "offsets": torch.empty(E + 1, dtype=i32, device=device),
        "sorted_src": torch.empty(TK, dtype=i32, device=device),
        "dest": torch.empty(TK, dtype=i32, device=device),
        "x_perm": torch.empty(TK, d, dtype=dt, device=device),
        "h": torch.empty(TK, f, dtype=dt, device=device),
        "y_perm": torch.empty(TK, d, dtype=dt, device=device),
        "y_shared": (torch.empty(T, d, dtype=dt, device=device)
                     if desc.d_ff_shared else None),
        "act_a": None, "act_b": None,
    }
    if desc.flags & B.MOE_FLAG_SAVE_ACTS:
        bufs["act_a"] = torch.empty(TK, f, dtype=dt, device=device)
        bufs["act_b"] = torch.empty(TK, f, dtype=dt, device=device)
    bufs["ws"] = torch.empty(max(B.moe_workspace_size(desc), 1),
                             dtype=torch.uint8, device=device)
    return bufs


def fwd_args(inp: dict, bufs: dict,
             events: Optional[Sequence] = None) -> B.MoeFwdArgs:
    a = B.MoeFwdArgs()
    p = B.ptr
    a.x = p(inp["x"])
    a.w_router = p(inp.get("wr"))
    a.route_bias = p(inp.get("bias"))
    a.logits_in = p(inp.get("logits_in"))
    a.routed = B.expert_weights(inp["w1"], inp["w3"], inp["w2"])
    a.shared = B.expert_weights(inp.get("ws1"), inp.get("ws3"), inp.get("ws2"))
    for k in ("out", "logits", "topk_idx", "topk_w", "counts", "offsets",
              "sorted_src", "dest", "x_perm", "h", "y_perm", "y_shared",
              "act_a", "act_b"):
        setattr(a, k, p(bufs.get(k)))
    if inp.get("logits_in") is not None:
        a.logits = None
    if events:
        for i, ev in enumerate(events[:B.MOE_FWD_NEVENTS]):
            a.events[i] = ev
    return a


def forward(desc: B.MoeDesc, inp: dict, bufs: dict, events=None,
            stream=None) -> torch.Tensor:
    B.moe_forward(desc, fwd_args(inp, bufs, events), bufs["ws"], stream)
    return bufs["out"]


def alloc_backward(desc: B.MoeDesc, device="cuda") -> dict:
    T, d, f, E, K = desc.T, desc.d_model, desc.d_ff, desc.E, desc.K
    dt = act_torch_dtype(desc)
    return {
        "dx": torch.empty(T, d, dtype=dt, device=device),
        "dw1": torch.empty(E, f, d, dtype=dt, device=device),
        "dw3": torch.empty(E, f, d, dtype=dt, device=device),
        "dw2": torch.empty(E, d, f, dtype=dt, device=device),
        "d_topk_w": torch.empty(T, K, dtype=torch.float32, device=device),
        "ws": torch.empty(max(B.moe_workspace_size(desc, True), 1),
                          dtype=torch.uint8, device=device),
    }


def bwd_args(inp: dict, fbufs: dict, dy: torch.Tensor, gbufs: dict,
             events=None) -> B.MoeBwdArgs:
    a = B.MoeBwdArgs()
    p = B.ptr
    a.dy = p(dy)
    a.x = p(inp["x"])
    a.routed = B.expert_weights(inp["w1"], inp["w3"], inp["w2"])
    a.shared = B.expert_weights(inp.get("ws1"), inp.get("ws3"), inp.get("ws2"))
    for k in ("topk_idx", "topk_w", "offsets", "sorted_src", "dest", "x_perm",
              "h", "y_perm", "act_a", "act_b"):
        setattr(a, k, p(fbufs.get(k)))
    for k in ("dx", "dw1", "dw3", "dw2", "d_topk_w"):
        setattr(a, k, p(gbufs[k]))
    if events:
        for i, ev in enumerate(events[:B.MOE_BWD_NEVENTS]):
            a.events[i] = ev
    return a


def backward(desc: B.MoeDesc, inp: dict, fbufs: dict, dy: torch.Tensor,
             gbufs: dict, events=None, stream=None) -> dict:
    B.moe_backward(desc, bwd_args(inp, fbufs, dy, gbufs, events), gbufs["ws"],
                   stream)
    return gbufs
