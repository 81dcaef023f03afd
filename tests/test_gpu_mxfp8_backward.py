"""MXFP8 backward on the GPU against the fp8-aware oracle backward
(max|err| / max|ref| <= 2e-2, as the MXFP8 forward): the data-gradient
products on MX operands quantised along their contraction, the weight
gradients from the forward's operands. Also the transposing weight
quantiser, code for code."""
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import DEV, check_routing_exact, inputs, rel_err
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

MX_TOL = 2e-2

CASES = [
    mi.MoEConfig("mxb_T1024_d256_f512_E8_K2", 1024, 256, 512, 8, 2),
    mi.MoEConfig("mxb_sigmoid_T512_d256_f256_E16_K4", 512, 256, 256, 16, 4,
                 gate="sigmoid", bias=True),
    mi.MoEConfig("mxb_tail_T333_d384_f256_E16_K3", 333, 384, 256, 16, 3),
    # >= 512 rows per expert on average: weight-gradient tiles of many
    # k-tiles, on the persistent kernel (empty experts in the skewed case)
    mi.MoEConfig("mxb_long_k_T2048_d256_f256_E4_K2", 2048, 256, 256, 4, 2),
    mi.MoEConfig("mxb_long_k_skewed_T4096_d128_f256_E16_K4", 4096, 128, 256,
                 16, 4, synth_logits=True, n_zero=3, zipf_s=1.2),
    mi.MoEConfig("mxb_skewed_T1024_d256_f256_E16_K4", 1024, 256, 256, 16, 4,
                 synth_logits=True, n_zero=3, zipf_s=1.2),
    mi.MoEConfig("mxb_shared_sigmoid_T512_d256_f128_E16_K4_fs256", 512, 256,
                 128, 16, 4, f_shared=256, gate="sigmoid", bias=True),
]


def test_transposing_quantiser_exact():
    g = torch.Generator().manual_seed(40)
    # R = 96 rows land at column 128 of a 256-wide destination: a partial
    # last span, and spans before and after that stay untouched
    E, R, C = 3, 96, 192
    src = (torch.randn(E, R, C, generator=g) * 2.0).to(torch.bfloat16)
    ldq, col = 256, 128
    q = torch.zeros(E, C, ldq, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(L.mx_scale_shape(E * C, ldq), dtype=torch.uint8, device=DEV)
    B.moe_quantize_mxfp8_t(src.to(DEV), E, R, C, q, sc, ldq, col)
    torch.cuda.synchronize()
    rows = L.mx_scales_rows(sc, (E, C)).cpu()
    for e in range(E):
        rq, rc = oracle.mx_quantize(src[e].double().T)
        assert torch.equal(rows[e, :, col // 32:(col + R) // 32], rc)
        codes = q[e, :, col:col + R].cpu().view(torch.float8_e4m3fn).double()
        assert torch.equal(codes, rq)
        assert (q[e, :, :col] == 0).all() and (q[e, :, col + R:] == 0).all()
        assert (rows[e, :, :col // 32] == 0).all()
        assert (rows[e, :, (col + R) // 32:] == 0).all()


def _mx_train(cfg, ginp, save_acts=False):
    desc = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, cfg.f_shared,
                       gate=cfg.gate, mxfp8=True, save_acts=save_acts)
    ginp = dict(ginp)
    ginp["mx"] = L.quantize_expert_weights(ginp)
    ginp["mx_bwd"] = L.quantize_expert_weights_bwd(ginp)
    fb = L.alloc_forward(desc, DEV)
    L.forward(desc, ginp, fb)
    gb = L.alloc_backward(desc, DEV)
    L.backward(desc, ginp, fb, ginp["dy"], gb)
    torch.cuda.synchronize()
    return fb, gb


@pytest.mark.parametrize("save_acts", [False, True],
                         ids=["recompute", "saved"])
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_mxfp8_backward_parity(cfg, save_acts):
    cinp, ginp = inputs(cfg, seed=6, with_dy=True)
    fb, gb = _mx_train(cfg, ginp, save_acts)
    idx, w, counts, *_ = check_routing_exact(cfg, cinp, fb)
    sh = (cinp["ws1"], cinp["ws3"], cinp["ws2"])
    ref = oracle.backward_mxfp8(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"],
                                idx, w, cinp["dy"], *sh)
    exact = oracle.backward(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"],
                            idx, w, cinp["dy"], *sh)
    keys = [("dx", "dx"), ("dw1", "dw1"), ("dw3", "dw3"), ("dw2", "dw2"),
            ("d_topk_w", "d_w")]
    if cfg.f_shared:
        keys += [("dws1", "dws1"), ("dws3", "dws3"), ("dws2", "dws2")]
    for k, rk in keys:
        err = rel_err(gb[k], ref[rk])
        print(f"{cfg.name} {k}: vs fp8-aware oracle {err:.3e}, vs exact "
              f"{rel_err(gb[k], exact[rk]):.3e}")
        assert err <= MX_TOL, (k, err)
    for e in (counts == 0).nonzero().flatten().tolist():
        assert (gb["dw1"][e] == 0).all() and (gb["dw2"][e] == 0).all()


def test_mxfp8_backward_full_size_sampled():
    """Mixtral-shaped MXFP8 training step: dX and d_topk_w on sampled
    tokens, dW1/dW3 rows and dW2 columns on sampled hidden units."""
    cfg = mi.MIXTRAL_TRAIN
    ginp = mi.make_inputs(cfg, 0, device=DEV, with_dy=True)
    fb, gb = _mx_train(cfg, ginp, save_acts=True)
    idx, w, *_ = check_routing_exact(cfg, {"logits_in": None, "bias": None,
                                      "x": ginp["x"], "wr": ginp["wr"]}, fb)
    g = torch.Generator().manual_seed(1)
    toks = [0, cfg.T - 1]
    e0 = int(idx[0, 0])
    cols = [(e0, int(torch.randint(0, cfg.f, (1,), generator=g))),
            (e0, cfg.f - 1)]
    ref = oracle.backward_mxfp8_sampled(ginp["x"], ginp["w1"], ginp["w3"],
                                        ginp["w2"], idx, w, ginp["dy"], toks,
                                        cols)
    t = torch.tensor(toks, device=DEV)
    assert rel_err(gb["dx"][t], ref["dx"]) <= MX_TOL
    assert rel_err(gb["d_topk_w"][t], ref["d_w"]) <= MX_TOL
    for i, (e, j) in enumerate(cols):
        assert rel_err(gb["dw1"][e, j], ref["dw1_rows"][i]) <= MX_TOL, (e, j)
        assert rel_err(gb["dw3"][e, j], ref["dw3_rows"][i]) <= MX_TOL, (e, j)
        assert rel_err(gb["dw2"][e, :, j], ref["dw2_cols"][i]) <= MX_TOL, (e, j)


def test_mxfp8_saved_acts_match_recompute():
    """The pre-activations the MX forward saves are the ones the backward
    recomputes: both backward paths give identical gradients, and the
    forward's output does not change when it saves them."""
    cfg = CASES[0]
    _, ginp = inputs(cfg, seed=7, with_dy=True)
    fr, gr = _mx_train(cfg, ginp, False)
    fs, gs = _mx_train(cfg, ginp, True)
    assert torch.equal(fr["out"], fs["out"])
    for k in ("dx", "dw1", "dw3", "dw2", "d_topk_w"):
        assert torch.equal(gr[k], gs[k]), k
