"""Helpers shared by the GPU parity tests: seeded inputs on both sides,
the HIP path through the C ABI, and comparison rules.

Inputs are drawn on the CPU from moe_inputs and copied to the GPU, so the
oracle and the kernels see identical values. The oracle is always fed the
GPU's own fp32 logits (selection is decided on the same fp32 numbers)."""
from __future__ import annotations

import torch

import moe_inputs as mi
import oracle
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

DEV = "cuda"


def tol(cfg) -> float:
    """max|gpu - ref| / max|ref| bound: 1e-4 for fp32 layers, 1e-2 for
    bf16 layers (values stored in bf16 carry a relative rounding of 2^-9)."""
    return 1e-4 if cfg.dtype == "f32" else 1e-2


def rel_err(gpu: torch.Tensor, ref: torch.Tensor) -> float:
    g = gpu.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    den = r.abs().max().item()
    return (g - r).abs().max().item() / (den if den > 0 else 1.0)


def desc_of(cfg, save_acts=False, T=None):
    return B.make_desc(cfg.T if T is None else T, cfg.d, cfg.f, cfg.E, cfg.K,
                       cfg.f_shared, cfg.gate, cfg.dtype, save_acts=save_acts)


def inputs(cfg, seed=0, with_dy=False, device_gen=False):
    """(cpu inputs, gpu inputs). device_gen draws large tensors on the GPU
    (its own generator) and copies them to the host instead."""
    if device_gen:
        g = mi.make_inputs(cfg, seed, device=DEV, with_dy=with_dy)
        c = {k: (v.cpu() if isinstance(v, torch.Tensor) and v.is_cuda else v)
             for k, v in g.items()}
        return c, g
    c = mi.make_inputs(cfg, seed, with_dy=with_dy)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
         for k, v in c.items()}
    return c, g


def run_forward(cfg, ginp, save_acts=False):
    desc = desc_of(cfg, save_acts)
    bufs = L.alloc_forward(desc, DEV)
    L.forward(desc, ginp, bufs)
    torch.cuda.synchronize()
    return desc, bufs


def oracle_routing(cfg, cinp, bufs):
    """Oracle routing from the GPU's logits (or the synthesised ones)."""
    logits = cinp["logits_in"] if cinp.get("logits_in") is not None \
        else bufs["logits"].cpu()
    return oracle.route(logits, cfg.K, cfg.gate, cinp.get("bias"))


def check_logits(cinp, bufs):
    """The device router logits against fp64 x Wr^T (the routing checks
    below route the oracle on the device's own logits, so they alone
    cannot see a wrong router GEMM)."""
    ref = oracle.router_logits(cinp["x"], cinp["wr"])
    err = rel_err(bufs["logits"], ref)
    assert err <= 1e-4, f"router logits rel err {err}"


def check_routing_exact(cfg, cinp, bufs):
    """Routing bit-exact against the oracle routed on the same logits; the
    logits themselves are checked whenever the router GEMM made them (every
    caller passes x and wr then)."""
    if cinp.get("logits_in") is None:
        assert "x" in cinp and "wr" in cinp, "pass x and wr to check the logits"
        check_logits(cinp, bufs)
    idx, w = oracle_routing(cfg, cinp, bufs)
    g_idx = bufs["topk_idx"].cpu().to(torch.int64)
    assert torch.equal(g_idx, idx), "topk_idx differs"
    g_w = bufs["topk_w"].cpu().double()
    werr = ((g_w - w).abs() / w.abs().clamp_min(1e-30)).max().item()
    assert werr <= 1e-6, f"topk_w rel err {werr}"
    counts, offsets, src, dest = oracle.permute(idx, cfg.E)
    assert torch.equal(bufs["counts"].cpu().long(), counts)
    assert torch.equal(bufs["offsets"].cpu().long(), offsets)
    assert torch.equal(bufs["sorted_src"].cpu().long(), src)
    assert torch.equal(bufs["dest"].cpu().long(), dest)
    return idx, w, counts, offsets, src, dest
