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


def is_mx(desc: B.MoeDesc) -> bool:
    return desc.gemm_dtype == B.MOE_MXFP8


def mx_scale_shape(rows: int, cols: int):
    """Shape of the E8M0 scales of an MX operand of `rows` (stacked) rows
    and `cols` columns in the library's layout: [cols/128, rows, 4], the
    four codes of one row's 128-column span side by side."""
    return (cols // 128, rows, 4)


def mx_scales_rows(sc: torch.Tensor, lead) -> torch.Tensor:
    """The same codes row by row: [*lead, cols/32] (a layout change only;
    lead = the operand's leading dimensions, e.g. (E, d_ff))."""
    spans, rows, _ = sc.shape
    return sc.permute(1, 0, 2).reshape(*lead, spans * 4)


def quantize_mxfp8(t: torch.Tensor):
    """MX-quantise a bf16 tensor along its last dimension on the device:
    (E4M3 codes as uint8 with t's shape, E8M0 scales of the stacked
    [numel / cols, cols] operand, shape mx_scale_shape)."""
    cols = t.shape[-1]
    rows = t.numel() // cols
    q = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    sc = torch.empty(mx_scale_shape(rows, cols), dtype=torch.uint8,
                     device=t.device)
    B.moe_quantize_mxfp8(t.contiguous(), rows, cols, q, sc)
    return q, sc


def quantize_expert_weights(inp: dict) -> dict:
    """MXFP8 copies of the routed expert weights (quantised once, along
    each matrix's rows = the contraction dimension of its GEMM)."""
    out = {}
    for k in ("w1", "w3", "w2", "ws1", "ws3", "ws2"):
        if inp.get(k) is not None:
            out[k], out[k + "_s"] = quantize_mxfp8(inp[k])
    return out


def _quantize_t(w1, w3, w2):
    """w2t [E, f, d] (W2^T, blocks along d) and w13t [E, d, 2f]
    ([W1^T | W3^T], blocks along f) with their E8M0 scales."""
    E, f, d = w1.shape
    dev, u8 = w1.device, torch.uint8
    w2t = torch.empty(E, f, d, dtype=u8, device=dev)
    w2t_s = torch.empty(mx_scale_shape(E * f, d), dtype=u8, device=dev)
    w13t = torch.empty(E, d, 2 * f, dtype=u8, device=dev)
    w13t_s = torch.empty(mx_scale_shape(E * d, 2 * f), dtype=u8, device=dev)
    B.moe_quantize_mxfp8_t(w2.contiguous(), E, d, f, w2t, w2t_s, d)
    for col, w in ((0, w1), (f, w3)):
        B.moe_quantize_mxfp8_t(w.contiguous(), E, f, d, w13t, w13t_s, 2 * f,
                               col)
    return w2t, w2t_s, w13t, w13t_s


def quantize_expert_weights_bwd(inp: dict) -> dict:
    """MXFP8 copies of the weights for the backward's transposed products:
    w2t, w13t (routed) and, with a shared expert, ws2t, ws13t (E = 1), each
    with its E8M0 scales (key + "_s")."""
    out = {}
    keys = [("", "w1", "w3", "w2"), ("s", "ws1", "ws3", "ws2")]
    for tag, k1, k3, k2 in keys:
        if inp.get(k1) is None:
            continue
        w1, w3, w2 = inp[k1], inp[k3], inp[k2]
        if w1.dim() == 2:
            w1, w3, w2 = w1[None], w3[None], w2[None]
        w2t, w2t_s, w13t, w13t_s = _quantize_t(w1, w3, w2)
        sq = (lambda t: t[0]) if tag else (lambda t: t)
        # (the scales of E = 1 stacked operands are those of the one)
        out[f"w{tag}2t"], out[f"w{tag}2t_s"] = sq(w2t), w2t_s
        out[f"w{tag}13t"], out[f"w{tag}13t_s"] = sq(w13t), w13t_s
    return out


def alloc_forward(desc: B.MoeDesc, device="cuda", gather=False) -> dict:
    """Every caller-owned forward buffer for ``desc`` plus the workspace.
    MXFP8: x_perm holds E4M3 codes with scales in x_perm_scales, and h
    holds E4M3 codes [T*K, d_ff] followed by E8M0 scales. gather=True
    leaves x_perm out: GEMM 1 then reads its rows from x through
    sorted_src (the permute writes only the indices)."""
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
        "act_a": None, "act_b": None, "x_perm_scales": None,
    }
    if is_mx(desc):
        u8 = torch.uint8
        bufs["x_perm"] = torch.empty(TK, d, dtype=u8, device=device)
        bufs["x_perm_scales"] = torch.empty(mx_scale_shape(TK, d), dtype=u8,
                                            device=device)
        bufs["h"] = torch.empty(TK * f + TK * (f // 32), dtype=u8, device=device)
    if gather:
        bufs["x_perm"] = bufs["x_perm_scales"] = None
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
    if inp.get("mx") is not None:
        m = inp["mx"]
        a.routed = B.expert_weights(m["w1"], m["w3"], m["w2"], m["w1_s"],
                                    m["w3_s"], m["w2_s"])
        a.shared = B.expert_weights(m.get("ws1"), m.get("ws3"), m.get("ws2"),
                                    m.get("ws1_s"), m.get("ws3_s"),
                                    m.get("ws2_s"))
    else:
        a.routed = B.expert_weights(inp["w1"], inp["w3"], inp["w2"])
        a.shared = B.expert_weights(inp.get("ws1"), inp.get("ws3"),
                                    inp.get("ws2"))
    for k in ("out", "logits", "topk_idx", "topk_w", "counts", "offsets",
              "sorted_src", "dest", "x_perm", "x_perm_scales", "h", "y_perm",
              "y_shared", "act_a", "act_b"):
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


def forward_noalloc(desc: B.MoeDesc, inp: dict, bufs: dict, events=None,
                    stream=None) -> torch.Tensor:
    """forward() without a workspace: the library's static device scratch
    serves instead (bufs["ws"] is not used)."""
    B.moe_forward_noalloc(desc, fwd_args(inp, bufs, events), stream)
    return bufs["out"]


def alloc_backward(desc: B.MoeDesc, device="cuda") -> dict:
    T, d, f, E, K = desc.T, desc.d_model, desc.d_ff, desc.E, desc.K
    fs = desc.d_ff_shared
    dt = act_torch_dtype(desc)
    return {
        "dx": torch.empty(T, d, dtype=dt, device=device),
        "dw1": torch.empty(E, f, d, dtype=dt, device=device),
        "dw3": torch.empty(E, f, d, dtype=dt, device=device),
        "dw2": torch.empty(E, d, f, dtype=dt, device=device),
        "d_topk_w": torch.empty(T, K, dtype=torch.float32, device=device),
        "ws": torch.empty(max(B.moe_workspace_size(desc, True), 1),
                          dtype=torch.uint8, device=device),
        **({"dws1": torch.empty(fs, d, dtype=dt, device=device),
            "dws3": torch.empty(fs, d, dtype=dt, device=device),
            "dws2": torch.empty(d, fs, dtype=dt, device=device)}
           if fs > 0 else {}),
    }


def bwd_args(inp: dict, fbufs: dict, dy: torch.Tensor, gbufs: dict,
             events=None) -> B.MoeBwdArgs:
    a = B.MoeBwdArgs()
    p = B.ptr
    a.dy = p(dy)
    a.x = p(inp["x"])
    mx = inp.get("mx")
    if mx is not None:  # MXFP8: the forward's MX weights and the backward's
        a.routed = B.expert_weights(mx["w1"], mx["w3"], mx["w2"], mx["w1_s"],
                                    mx["w3_s"], mx["w2_s"])
        bw = inp["mx_bwd"]
        a.w2t, a.w2t_scales = p(bw["w2t"]), p(bw["w2t_s"])
        a.w13t, a.w13t_scales = p(bw["w13t"]), p(bw["w13t_s"])
        if "ws1" in mx:
            a.shared = B.expert_weights(mx["ws1"], mx["ws3"], mx["ws2"],
                                        mx["ws1_s"], mx["ws3_s"], mx["ws2_s"])
            a.ws2t, a.ws2t_scales = p(bw["ws2t"]), p(bw["ws2t_s"])
            a.ws13t, a.ws13t_scales = p(bw["ws13t"]), p(bw["ws13t_s"])
    else:
        a.routed = B.expert_weights(inp["w1"], inp["w3"], inp["w2"])
        a.shared = B.expert_weights(inp.get("ws1"), inp.get("ws3"),
                                    inp.get("ws2"))
    for k in ("topk_idx", "topk_w", "offsets", "sorted_src", "dest", "x_perm",
              "h", "y_perm", "act_a", "act_b", "x_perm_scales"):
        setattr(a, k, p(fbufs.get(k)))
    for k in ("dx", "dw1", "dw3", "dw2", "d_topk_w", "dws1", "dws3", "dws2"):
        setattr(a, k, p(gbufs.get(k)))
    if events:
        for i, ev in enumerate(events[:B.MOE_BWD_NEVENTS]):
            a.events[i] = ev
    return a


def backward(desc: B.MoeDesc, inp: dict, fbufs: dict, dy: torch.Tensor,
             gbufs: dict, events=None, stream=None) -> dict:
    B.moe_backward(desc, bwd_args(inp, fbufs, dy, gbufs, events), gbufs["ws"],
                   stream)
    return gbufs


def alloc_router_backward(desc: B.MoeDesc, device="cuda") -> dict:
    T, d, E = desc.T, desc.d_model, desc.E
    dt = act_torch_dtype(desc)
    return {
        "d_logits": torch.empty(T, E, dtype=torch.float32, device=device),
        "d_w_router": torch.empty(E, d, dtype=dt, device=device),
        "ws": torch.empty(max(B.moe_router_workspace_size(desc), 1),
                          dtype=torch.uint8, device=device),
        "f": torch.empty(E, dtype=torch.float32, device=device),
        "p_mean": torch.empty(E, dtype=torch.float32, device=device),
        "aux": torch.empty(1, dtype=torch.float32, device=device),
    }


def load_balance_stats(desc: B.MoeDesc, fbufs: dict, rbufs: dict,
                       stream=None) -> dict:
    """After forward(): the balance statistics of its routing into
    rbufs["f"], rbufs["p_mean"] and rbufs["aux"]."""
    B.moe_load_balance_stats(desc, fbufs["logits"], fbufs["counts"],
                             rbufs["f"], rbufs["p_mean"], rbufs["aux"],
                             rbufs["ws"], stream)
    return rbufs


def router_backward(desc: B.MoeDesc, inp: dict, fbufs: dict, gbufs: dict,
                    rbufs: dict, aux_coef: float = 0.0, stream=None) -> dict:
    """After backward(): carries gbufs["d_topk_w"] (and, with aux_coef,
    the balance loss) through the gate into rbufs["d_logits"] and
    rbufs["d_w_router"], and adds the router's share of the input
    gradient into gbufs["dx"]."""
    B.moe_router_backward(desc, inp["x"], inp["wr"], fbufs["logits"],
                          fbufs["topk_idx"], fbufs["topk_w"],
                          gbufs["d_topk_w"], fbufs["counts"], aux_coef,
                          rbufs["d_logits"], rbufs["d_w_router"], gbufs["dx"],
                          rbufs["ws"], stream)
    return rbufs
