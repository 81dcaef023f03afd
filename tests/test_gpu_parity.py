"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Routing, counts, offsets, permutation and x_perm must be bit-exact given
the same fp32 logits; gate weights within 1e-6 relative; floating-point
outputs within max|err|/max|ref| <= 1e-2 (bf16) or 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import (DEV, check_routing_exact, desc_of, inputs,
                         rel_err, run_forward, tol)
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

# Small workloads the oracle finishes in seconds; each spans several tiles
# and has ragged tails. Shapes mirror the full workloads' structure.
SMALL = [
    mi.TINY_FP32,
    # ~512 rows per expert: big tiles whose ragged last tile skips its
    # empty 32-row blocks (groups below 1024 rows)
    mi.MoEConfig("mixtral_like_T2048_d256_f512_E8_K2", 2048, 256, 512, 8, 2),
    mi.MoEConfig("mixtral_like_f32_T512_d128_f192_E8_K2", 512, 128, 192, 8, 2,
                 dtype="f32"),
    mi.MoEConfig("deepseek_like_T256_d512_f256_E64_K8_shared", 256, 512, 256,
                 64, 8, f_shared=256, gate="sigmoid", bias=True),
    mi.MoEConfig("skewed_like_T2048_d256_f128_E32_K4", 2048, 256, 128, 32, 4,
                 synth_logits=True, n_zero=4, zipf_s=1.2),
    # ~128 rows per expert, as in the DeepSeek-V3 shape: one 256-row tile
    # per expert with the empty 32-row blocks' MFMAs skipped
    mi.MoEConfig("deepseek_mid_rows_T1024_d256_f256_E64_K8_shared", 1024, 256,
                 256, 64, 8, f_shared=256, gate="sigmoid", bias=True),
    # expert counts that are not a multiple of 8: the router GEMM's last
    # 8-column output piece of a row is partial (E = 4, 60) or its rows
    # are not 16-byte aligned (E = 6); E = 60 with a shared expert is the
    # Qwen-MoE-like structure
    mi.MoEConfig("four_experts_T1024_d128_f128_E4_K2", 1024, 128, 128, 4, 2),
    mi.MoEConfig("six_experts_T1024_d256_f256_E6_K2", 1024, 256, 256, 6, 2),
    mi.MoEConfig("qwen_like_T1024_d256_f192_E60_K4_shared384", 1024, 256, 192,
                 60, 4, f_shared=384),
    # widths that are multiples of 8 but not of 64: the register-staged
    # MFMA kernel (k-tiles zero-filled past K) for every forward product
    mi.MoEConfig("narrow_T512_d200_f328_E8_K2", 512, 200, 328, 8, 2),
    mi.MoEConfig("narrow_shared_T256_d136_f200_E6_K2_fs72", 256, 136, 200, 6,
                 2, f_shared=72),
    # the library's limits: E = 1024 experts, K = 16 per token (about 8
    # rows per expert, some experts empty)
    mi.MoEConfig("max_experts_T512_d128_f64_E1024_K16", 512, 128, 64, 1024,
                 16),
]
IDS = [c.name for c in SMALL]


def _oracle_forward(cfg, cinp, idx, w, tokens=None):
    return oracle.forward(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"], idx,
                          w, cinp["ws1"], cinp["ws3"], cinp["ws2"],
                          tokens=tokens)


@pytest.mark.parametrize("cfg", SMALL, ids=IDS)
def test_forward_parity(cfg):
    cinp, ginp = inputs(cfg, seed=0)
    desc, bufs = run_forward(cfg, ginp)
    idx, w, counts, offsets, src, dest = check_routing_exact(cfg, cinp, bufs)
    if cinp.get("logits_in") is None:
        ref_logits = oracle.router_logits(cinp["x"], cinp["wr"])
        assert rel_err(bufs["logits"], ref_logits) <= 1e-4
    else:
        assert torch.equal(counts, cinp["loads"])
    # x_perm is an exact copy
    assert torch.equal(bufs["x_perm"].cpu(), cinp["x"][src // cfg.K])
    ref = _oracle_forward(cfg, cinp, idx, w)
    err = rel_err(bufs["out"], ref)
    assert err <= tol(cfg), f"out rel err {err}"


@pytest.mark.parametrize("cfg", SMALL, ids=IDS)
def test_stage_parity(cfg):
    """Each GEMM and the combine against the oracle on the GPU's own inputs."""
    cinp, ginp = inputs(cfg, seed=1)
    desc, bufs = run_forward(cfg, ginp, save_acts=True)
    offsets = bufs["offsets"].cpu()
    a, b, h = oracle.stage_gemm1(bufs["x_perm"].cpu(), offsets, cinp["w1"],
                                 cinp["w3"])
    assert rel_err(bufs["h"], h) <= tol(cfg)
    assert rel_err(bufs["act_a"], a) <= tol(cfg)
    assert rel_err(bufs["act_b"], b) <= tol(cfg)
    y = oracle.stage_gemm2(bufs["h"].cpu(), offsets, cinp["w2"])
    assert rel_err(bufs["y_perm"], y) <= tol(cfg)
    ysh = bufs["y_shared"].cpu() if bufs["y_shared"] is not None else None
    if ysh is not None:
        ref_sh = oracle.expert_ffn(cinp["x"], cinp["ws1"], cinp["ws3"],
                                   cinp["ws2"])[3]
        assert rel_err(ysh, ref_sh) <= tol(cfg)
    out = oracle.stage_combine(bufs["y_perm"].cpu(), bufs["dest"].cpu(),
                               bufs["topk_w"].cpu(), ysh)
    assert rel_err(bufs["out"], out) <= (1e-6 if cfg.dtype == "f32" else 4e-3)


def test_tie_logits_routing_exact():
    for gate in ("softmax", "sigmoid"):
        for E, K in ((8, 2), (64, 8), (130, 5), (256, 8), (1024, 16)):
            cfg = mi.MoEConfig("ties", 200, 64, 64, E, K, gate=gate,
                               synth_logits=True)
            logits = mi.tie_logits(200, E)
            bias = (torch.rand(E, generator=torch.Generator().manual_seed(E))
                    * 0.2 - 0.1) if gate == "sigmoid" else None
            desc = desc_of(cfg)
            idx = torch.empty(200, K, dtype=torch.int32, device=DEV)
            w = torch.empty(200, K, dtype=torch.float32, device=DEV)
            B.moe_route(desc, None, None,
                        bias.to(DEV) if bias is not None else None,
                        logits.to(DEV), None, idx, w)
            torch.cuda.synchronize()
            ridx, rw = oracle.route(logits, K, gate, bias)
            assert torch.equal(idx.cpu().long(), ridx), (gate, E, K)
            werr = ((w.cpu().double() - rw).abs() / rw).max().item()
            assert werr <= 1e-6, (gate, E, K, werr)


def _forward_with_logits(cfg, logits, seed=3):
    cinp, ginp = inputs(cfg.replace(synth_logits=False), seed=seed)
    cinp["logits_in"] = logits
    ginp["logits_in"] = logits.to(DEV)
    desc, bufs = run_forward(cfg, ginp)
    return cinp, bufs


def _logits_for_loads(T, E, K, assign):
    """fp32 logits whose top-K rows are exactly `assign` [T, K]."""
    lg = torch.full((T, E), -1.0)
    for k in range(K):
        lg[torch.arange(T), assign[:, k]] = 2.0 + (K - k) * 0.25
    return lg


@pytest.mark.parametrize("case", [
    "all_to_one", "empty_middle", "tile_edges_128", "tile_edges_256",
    "single_token", "k_equals_e", "single_expert"])
def test_edge_routing(case):
    T, d, f, E, K = 640, 128, 256, 6, 1
    if case == "all_to_one":
        assign = torch.full((T, 1), 3)
    elif case == "empty_middle":
        assign = torch.randint(0, E, (T, 1), generator=torch.Generator().manual_seed(0))
        assign[assign == 2] = 4
    elif case in ("tile_edges_128", "tile_edges_256"):
        bm = 128 if case.endswith("128") else 256
        loads = [1, bm - 1, bm, bm + 1, 0]
        if bm == 256:  # one large expert lifts rows/expert to 256-row tiles
            loads.append(1000)
            d, f = 256, 512
        E = len(loads)
        T = sum(loads)
        assign = torch.tensor(np.repeat(np.arange(E), loads))[:, None]
    elif case == "single_token":
        T, E, K = 1, 8, 2
        assign = torch.tensor([[5, 1]])
    elif case == "k_equals_e":
        T, E, K = 96, 4, 4
        assign = torch.tensor([[2, 0, 3, 1]] * T)
    else:
        T, E, K = 300, 1, 1
        assign = torch.zeros((T, 1), dtype=torch.long)
    cfg = mi.MoEConfig(case, T, d, f, E, K, synth_logits=True)
    cinp, bufs = _forward_with_logits(cfg, _logits_for_loads(T, E, K, assign))
    idx, w, counts, offsets, src, dest = check_routing_exact(cfg, cinp, bufs)
    assert torch.equal(idx, assign.long())
    ref = _oracle_forward(cfg, cinp, idx, w)
    assert rel_err(bufs["out"], ref) <= tol(cfg)


def test_combine_k1_w1_is_bit_exact():
    T, E = 700, 7
    cfg = mi.MoEConfig("k1", T, 128, 128, E, 1, synth_logits=True)
    assign = torch.randint(0, E, (T, 1), generator=torch.Generator().manual_seed(1))
    cinp, bufs = _forward_with_logits(cfg, _logits_for_loads(T, E, 1, assign))
    assert (bufs["topk_w"].cpu() == 1.0).all()
    y = bufs["y_perm"].cpu()
    dest = bufs["dest"].cpu().long()
    assert torch.equal(bufs["out"].cpu(), y[dest])


def test_zero_tokens_is_a_no_op():
    cfg = mi.MoEConfig("empty", 0, 128, 128, 4, 2)
    desc = desc_of(cfg)
    bufs = L.alloc_forward(desc, DEV)
    x = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    w = torch.empty(4, 128, 128, dtype=torch.bfloat16, device=DEV)
    L.forward(desc, {"x": x, "wr": w[:, 0], "w1": w, "w3": w, "w2": w}, bufs)
    torch.cuda.synchronize()


def test_determinism():
    cfg = SMALL[4]
    cinp, ginp = inputs(cfg, seed=5)
    _, b1 = run_forward(cfg, ginp)
    _, b2 = run_forward(cfg, ginp)
    for k in ("out", "h", "y_perm", "x_perm", "dest", "topk_w"):
        assert torch.equal(b1[k], b2[k]), k


def test_hip_graph_replay_with_new_routing():
    """Capture the whole forward once; replay it with inputs whose expert
    loads differ every time (including empty experts). No host sync and
    no shape recompile are needed for the replay to stay correct."""
    cfg = mi.MoEConfig("graph_T1024_d256_f256_E16_K4", 1024, 256, 256, 16, 4,
                       synth_logits=True, n_zero=3, zipf_s=1.2)
    cinp, ginp = inputs(cfg, seed=0)
    desc = desc_of(cfg)
    bufs = L.alloc_forward(desc, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.forward(desc, ginp, bufs)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(desc, ginp, bufs)
    for rep in range(4):
        n_zero = [0, 5, 2, 9][rep]
        lg, loads = mi.synth_logits(cfg.T, cfg.E, cfg.K, n_zero, 1.0 + 0.3 * rep,
                                    seed=10 + rep)
        x = mi.randn((cfg.T, cfg.d), 1.0, 20 + rep, "x", torch.bfloat16)
        ginp["logits_in"].copy_(lg.to(DEV))
        ginp["x"].copy_(x.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["counts"].cpu().long(), loads)
        cinp["logits_in"], cinp["x"] = lg, x
        idx, w, *_ = check_routing_exact(cfg, cinp, bufs)
        ref = _oracle_forward(cfg, cinp, idx, w)
        assert rel_err(bufs["out"], ref) <= tol(cfg), rep
        # eager work between replays
        torch.zeros(1024, device=DEV).sum().item()
