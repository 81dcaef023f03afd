"""A whole training step (forward with saved activations, balance
statistics, backward, router backward with the balance loss) captured once
in a HIP graph and replayed on new tokens and new routing: every replay
must equal the same step run eagerly, bit for bit. Eager work and host
synchronisations run between the replays. Also the MXFP8 training step."""
import pytest
import torch

import moe_inputs as mi
from moe_testlib import DEV, desc_of, inputs
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

OUTS_F = ("out", "counts", "topk_idx")
OUTS_G = ("dx", "dw1", "dw3", "dw2", "d_topk_w")
OUTS_R = ("d_logits", "d_w_router", "f", "p_mean", "aux")


def _alloc(desc):
    return (L.alloc_forward(desc, DEV), L.alloc_backward(desc, DEV),
            L.alloc_router_backward(desc, DEV))


def _step(desc, inp, bufs, router=True):
    fb, gb, rb = bufs
    L.forward(desc, inp, fb)
    if router:
        L.load_balance_stats(desc, fb, rb)
    L.backward(desc, inp, fb, inp["dy"], gb)
    if router:
        L.router_backward(desc, inp, fb, gb, rb, aux_coef=0.01)


def _replay_check(desc, ginp, new_inputs, router=True):
    graph_bufs = _alloc(desc)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(desc, ginp, graph_bufs, router)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(desc, ginp, graph_bufs, router)
    eager_bufs = _alloc(desc)
    for rep, (x, dy) in enumerate(new_inputs):
        ginp["x"].copy_(x)
        ginp["dy"].copy_(dy)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _step(desc, ginp, eager_bufs, router)
        torch.cuda.synchronize()
        fb, gb, rb = graph_bufs
        efb, egb, erb = eager_bufs
        for k in OUTS_F:
            assert torch.equal(fb[k], efb[k]), (rep, k)
        for k in OUTS_G:
            assert torch.equal(gb[k], egb[k]), (rep, k)
        if router:
            for k in OUTS_R:
                assert torch.equal(rb[k], erb[k]), (rep, k)
        torch.zeros(1024, device=DEV).sum().item()  # eager work between


def _new_inputs(cfg, n):
    out = []
    for rep in range(n):
        x = mi.randn((cfg.T, cfg.d), 1.0 + 0.5 * rep, 40 + rep, "x",
                     torch.bfloat16).to(DEV)
        dy = mi.randn((cfg.T, cfg.d), 1.0, 50 + rep, "dy",
                      torch.bfloat16).to(DEV)
        out.append((x, dy))
    return out


def test_training_step_graph_replay():
    cfg = mi.MoEConfig("graph_train_T512_d256_f256_E16_K4_sigmoid", 512, 256,
                       256, 16, 4, gate="sigmoid", bias=True)
    _, ginp = inputs(cfg, seed=0, with_dy=True)
    desc = desc_of(cfg, save_acts=True)
    _replay_check(desc, ginp, _new_inputs(cfg, 3))


def test_mxfp8_training_step_graph_replay():
    cfg = mi.MoEConfig("graph_mx_train_T512_d256_f256_E8_K2", 512, 256, 256,
                       8, 2)
    _, ginp = inputs(cfg, seed=1, with_dy=True)
    desc = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, 0, gate=cfg.gate,
                       mxfp8=True, save_acts=True)
    ginp = dict(ginp)
    ginp["mx"] = L.quantize_expert_weights(ginp)
    ginp["mx_bwd"] = L.quantize_expert_weights_bwd(ginp)
    torch.cuda.synchronize()
    _replay_check(desc, ginp, _new_inputs(cfg, 3))
