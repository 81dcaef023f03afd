"""Router backward on the GPU against the oracle's closed-form gate
Jacobian: d_logits (fp32) within 1e-4 of max|ref|; the router-weight
gradient and the router's share of dx within the layer tolerance (they are
formed from d_logits rounded to the activation dtype). The share of dx is
added into the caller's dx: checked from zero and from a random dx."""
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import DEV, inputs, rel_err, run_forward, tol
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

CASES = [
    mi.TINY_FP32,
    mi.MoEConfig("rb_T1024_d256_f256_E8_K2", 1024, 256, 256, 8, 2),
    mi.MoEConfig("rb_T777_d384_f256_E16_K4", 777, 384, 256, 16, 4),
    mi.MoEConfig("rb_sigmoid_bias_T512_d256_f128_E32_K4", 512, 256, 128, 32, 4,
                 gate="sigmoid", bias=True),
]


def _run(cfg, seed, dx0_scale):
    cinp, ginp = inputs(cfg, seed)
    desc, fb = run_forward(cfg, ginp)
    g = torch.Generator().manual_seed(seed + 99)
    d_w = torch.randn(cfg.T, cfg.K, generator=g)
    dx0 = (torch.randn(cfg.T, cfg.d, generator=g) * dx0_scale).to(cfg.torch_dtype)
    gb = {"d_topk_w": d_w.to(DEV), "dx": dx0.to(DEV)}
    rb = L.alloc_router_backward(desc, DEV)
    L.router_backward(desc, ginp, fb, gb, rb)
    torch.cuda.synchronize()
    logits = fb["logits"].cpu()
    idx = fb["topk_idx"].cpu().long()
    w = fb["topk_w"].cpu()
    ref = oracle.router_backward(cinp["x"], cinp["wr"], logits, idx, w, d_w,
                                 cfg.gate)
    rb["_idx"] = idx
    return cfg, dx0, gb, rb, ref


def gb_idx(rb, cfg):
    return rb["_idx"]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_router_backward_parity(cfg):
    cfg, dx0, gb, rb, ref = _run(cfg, 5, 0.0)
    assert rel_err(rb["d_logits"], ref["d_logits"]) <= 1e-4
    assert rel_err(rb["d_w_router"], ref["d_wr"]) <= tol(cfg)
    assert rel_err(gb["dx"], ref["dx"]) <= tol(cfg)
    # zero gradient off the selection, exactly
    off = torch.ones(cfg.T, cfg.E, dtype=torch.bool)
    off.scatter_(1, gb_idx(rb, cfg), False)
    assert torch.all(rb["d_logits"].cpu()[off] == 0)


def test_router_backward_accumulates_into_dx():
    cfg = CASES[1]
    cfg, dx0, gb, rb, ref = _run(cfg, 6, 1.0)
    want = dx0.double() + ref["dx"]
    assert rel_err(gb["dx"], want) <= tol(cfg)


def test_router_backward_full_size_mixtral():
    """Mixtral-shaped layer: d_logits and the router-weight gradient whole,
    the share of dx on sampled tokens."""
    cfg = mi.MIXTRAL
    ginp = mi.make_inputs(cfg, 0, device=DEV)
    desc, fb = run_forward(cfg, ginp)
    g = torch.Generator().manual_seed(7)
    d_w = torch.randn(cfg.T, cfg.K, generator=g)
    gb = {"d_topk_w": d_w.to(DEV),
          "dx": torch.zeros(cfg.T, cfg.d, dtype=cfg.torch_dtype, device=DEV)}
    rb = L.alloc_router_backward(desc, DEV)
    L.router_backward(desc, ginp, fb, gb, rb)
    torch.cuda.synchronize()
    logits, idx, w = fb["logits"].cpu(), fb["topk_idx"].cpu().long(), fb["topk_w"].cpu()
    dl = oracle.gate_logit_grad(logits, idx, w, d_w, cfg.gate)
    assert rel_err(rb["d_logits"], dl) <= 1e-4
    x = ginp["x"].cpu().double()
    assert rel_err(rb["d_w_router"], dl.T @ x) <= tol(cfg)
    toks = torch.tensor([0, 1, 4095, cfg.T - 1])
    ref_dx = dl[toks] @ ginp["wr"].cpu().double()
    assert rel_err(gb["dx"][toks.to(DEV)], ref_dx) <= tol(cfg)


# ------------------------------------------------ load-balance statistics

def _stats_ref(logits, counts, idx, E, gate):
    ref = oracle.load_balance_stats(logits, idx, E, gate)
    # the oracle's share comes from the mask; counts must describe the same
    assert torch.equal(torch.bincount(idx.reshape(-1), minlength=E),
                       counts.long())
    return ref


def _check_stats(rb, ref):
    # f = counts / T: one correctly rounded fp32 division of exact integers
    assert torch.equal(rb["f"].cpu(), ref["f"].to(torch.float32))
    assert rel_err(rb["p_mean"], ref["p_mean"]) <= 1e-5
    assert abs(float(rb["aux"].cpu()[0]) - float(ref["aux"])) <= \
        1e-5 * abs(float(ref["aux"]))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_balance_stats_parity(cfg):
    cinp, ginp = inputs(cfg, 8)
    desc, fb = run_forward(cfg, ginp)
    rb = L.alloc_router_backward(desc, DEV)
    L.load_balance_stats(desc, fb, rb)
    torch.cuda.synchronize()
    idx = fb["topk_idx"].cpu().long()
    ref = _stats_ref(fb["logits"].cpu(), fb["counts"].cpu(), idx, cfg.E,
                     cfg.gate)
    _check_stats(rb, ref)


@pytest.mark.parametrize("T,E,K,gate", [(8192, 8, 2, "softmax"),
                                        (4096, 256, 8, "sigmoid"),
                                        (16384, 128, 8, "softmax"),
                                        (3, 1024, 16, "sigmoid")])
def test_balance_stats_full_size(T, E, K, gate):
    """The statistics at the Mixtral-, DeepSeek-V3- and skewed-shaped
    routing sizes (and the widest E with fewer tokens than waves), from
    seeded logits with their own selection and counts."""
    g = torch.Generator().manual_seed(T + E)
    logits = 1.5 * torch.randn(T, E, generator=g)
    idx = oracle.topk_select(oracle.selection_keys(logits), K)
    counts = torch.bincount(idx.reshape(-1), minlength=E).to(torch.int32)
    desc = L.B.make_desc(T, 256, 256, E, K, gate=gate)
    rb = L.alloc_router_backward(desc, DEV)
    fb = {"logits": logits.to(DEV), "counts": counts.to(DEV)}
    L.load_balance_stats(desc, fb, rb)
    torch.cuda.synchronize()
    _check_stats(rb, _stats_ref(logits, counts, idx, E, gate))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_aux_loss_backward_parity(cfg):
    """With d_topk_w = 0 the logit gradient is the balance loss's alone
    (its scale, coef * E / T, is far below the gate term, so it is checked
    on its own); then both terms together."""
    cinp, ginp = inputs(cfg, 9)
    desc, fb = run_forward(cfg, ginp)
    logits = fb["logits"].cpu()
    idx = fb["topk_idx"].cpu().long()
    w = fb["topk_w"].cpu()
    for coef, dw_scale in ((1.0, 0.0), (0.05, 1.0)):
        g = torch.Generator().manual_seed(10)
        d_w = torch.randn(cfg.T, cfg.K, generator=g) * dw_scale
        gb = {"d_topk_w": d_w.to(DEV),
              "dx": torch.zeros(cfg.T, cfg.d, dtype=cfg.torch_dtype,
                                device=DEV)}
        rb = L.alloc_router_backward(desc, DEV)
        L.router_backward(desc, ginp, fb, gb, rb, aux_coef=coef)
        torch.cuda.synchronize()
        ref = oracle.router_backward(cinp["x"], cinp["wr"], logits, idx, w,
                                     d_w, cfg.gate, aux_coef=coef)
        assert rel_err(rb["d_logits"], ref["d_logits"]) <= 1e-4
        assert rel_err(rb["d_w_router"], ref["d_wr"]) <= tol(cfg)
        assert rel_err(gb["dx"], ref["dx"]) <= tol(cfg)
