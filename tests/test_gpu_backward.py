"""Backward parity: dX, dW1, dW3, dW2 and the gate-weight gradients from
the HIP path against the oracle's closed-form backward (routing fixed,
gate weights as leaves). Small shapes in full; the Mixtral-shaped
training step on sampled tokens and hidden columns."""
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import (DEV, check_routing_exact, desc_of, inputs, rel_err,
                         tol)
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

CASES = [
    mi.TINY_FP32,
    mi.MoEConfig("mixtral_like_T1024_d256_f512_E8_K2", 1024, 256, 512, 8, 2),
    mi.MoEConfig("mixtral_like_f32_T256_d128_f96_E4_K2", 256, 128, 96, 4, 2,
                 dtype="f32"),
    mi.MoEConfig("skewed_like_T1024_d128_f192_E16_K4", 1024, 128, 192, 16, 4,
                 synth_logits=True, n_zero=3, zipf_s=1.2),
    # >= 512 rows per expert on average: weight-gradient tiles of many
    # k-tiles (ragged N with f = 192; empty experts in the skewed case)
    mi.MoEConfig("long_k_T2048_d256_f192_E4_K2", 2048, 256, 192, 4, 2),
    mi.MoEConfig("long_k_skewed_T4096_d128_f256_E16_K4", 4096, 128, 256, 16,
                 4, synth_logits=True, n_zero=3, zipf_s=1.2),
    mi.MoEConfig("many_experts_T256_d256_f128_E64_K8_sigmoid", 256, 256, 128,
                 64, 8, gate="sigmoid", bias=True),
    # ~128 rows per expert: the data-gradient products run one 256-row
    # tile per expert with the empty 32-row blocks' MFMAs skipped
    mi.MoEConfig("mid_rows_T1024_d256_f256_E16_K2", 1024, 256, 256, 16, 2),
    # widths that are multiples of 8 but not of 64: register-staged MFMA
    # products, and the SIMT kernel for dgrad1 (d_ff % 64 != 0)
    mi.MoEConfig("narrow_T512_d200_f328_E8_K2", 512, 200, 328, 8, 2),
    # the library's limits: E = 1024, K = 16 (some experts empty)
    mi.MoEConfig("max_experts_T256_d128_f64_E1024_K16", 256, 128, 64, 1024,
                 16),
    # E = 6: the router's output rows are not 16-byte aligned
    mi.MoEConfig("six_experts_T1024_d128_f192_E6_K2", 1024, 128, 192, 6, 2),
    # the persistent weight-gradient kernel (256 x 256 tiles) with partial
    # row and column tiles (d = 320, f = 264), empty experts (zero
    # gradients from a k-tile of zeros), experts of one to several k-tiles
    # (Zipf loads) and 320 tiles per product, more than one per workgroup
    mi.MoEConfig("wgrad_persist_T1024_d320_f264_E80_K2", 1024, 320, 264, 80,
                 2, synth_logits=True, n_zero=3, zipf_s=1.2),
    # ~256 rows per expert: the data gradients on 256 x 256 tiles reading
    # the weights k-major, each with a partial last column tile (dgrad2:
    # N = f = 448, dgrad1: N = d = 320) whose DMA chunks past N are clamped
    mi.MoEConfig("kmajor_ragged_n_T1024_d320_f448_E8_K2", 1024, 320, 448, 8,
                 2),
    # groups averaging 256 rows: the persistent weight-gradient kernel with
    # its DMA from half of the waves, 288 tiles per product (more than one
    # per workgroup on 256 CUs), partial row and column tiles (d = 576,
    # f = 520), Zipf loads and empty experts
    mi.MoEConfig("wgrad_half_dma_T4096_d576_f520_E32_K2", 4096, 576, 520, 32,
                 2, synth_logits=True, n_zero=3, zipf_s=1.2),
]


def _run(cfg, cinp, ginp, save_acts):
    desc = desc_of(cfg, save_acts=save_acts)
    fb = L.alloc_forward(desc, DEV)
    L.forward(desc, ginp, fb)
    gb = L.alloc_backward(desc, DEV)
    L.backward(desc, ginp, fb, ginp["dy"], gb)
    torch.cuda.synchronize()
    return fb, gb


@pytest.mark.parametrize("save_acts", [True, False], ids=["saved", "recompute"])
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_backward_parity(cfg, save_acts):
    cinp, ginp = inputs(cfg, seed=2, with_dy=True)
    fb, gb = _run(cfg, cinp, ginp, save_acts)
    idx, w, counts, *_ = check_routing_exact(cfg, cinp, fb)
    ref = oracle.backward(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"], idx,
                          w, cinp["dy"])
    for k, rk in (("dx", "dx"), ("dw1", "dw1"), ("dw3", "dw3"),
                  ("dw2", "dw2"), ("d_topk_w", "d_w")):
        err = rel_err(gb[k], ref[rk])
        assert err <= tol(cfg), (k, err)
    # experts that received no token get exactly zero gradient
    for e in (counts == 0).nonzero().flatten().tolist():
        assert (gb["dw1"][e] == 0).all() and (gb["dw2"][e] == 0).all()


SHARED = [
    mi.MoEConfig("shared_deepseek_like_T512_d256_f128_E16_K4_fs256", 512, 256,
                 128, 16, 4, f_shared=256, gate="sigmoid", bias=True),
    mi.MoEConfig("shared_f32_T128_d64_f64_E4_K2_fs96", 128, 64, 64, 4, 2,
                 f_shared=96, dtype="f32"),
    # Qwen-MoE-like structure: 60 fine-grained experts, top-4 softmax, an
    # ungated shared expert twice the routed width
    mi.MoEConfig("qwen_like_T1024_d256_f192_E60_K4_fs384", 1024, 256, 192, 60,
                 4, f_shared=384),
    # odd widths with a shared expert (staged MFMA and SIMT products)
    mi.MoEConfig("narrow_shared_T256_d136_f200_E6_K2_fs72", 256, 136, 200, 6,
                 2, f_shared=72),
]


@pytest.mark.parametrize("save_acts", [True, False], ids=["saved", "recompute"])
@pytest.mark.parametrize("cfg", SHARED, ids=[c.name for c in SHARED])
def test_backward_shared_expert(cfg, save_acts):
    """With an ungated shared expert: its weight gradients, and dx holding
    both the routed and the shared share."""
    cinp, ginp = inputs(cfg, seed=3, with_dy=True)
    fb, gb = _run(cfg, cinp, ginp, save_acts)
    idx, w, *_ = check_routing_exact(cfg, cinp, fb)
    ref = oracle.backward(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"], idx,
                          w, cinp["dy"], cinp["ws1"], cinp["ws3"], cinp["ws2"])
    for k, rk in (("dx", "dx"), ("dw1", "dw1"), ("dw3", "dw3"), ("dw2", "dw2"),
                  ("d_topk_w", "d_w"), ("dws1", "dws1"), ("dws3", "dws3"),
                  ("dws2", "dws2")):
        err = rel_err(gb[k], ref[rk])
        assert err <= tol(cfg), (k, err)


def test_backward_deterministic():
    cfg = CASES[3]
    cinp, ginp = inputs(cfg, seed=4, with_dy=True)
    _, g1 = _run(cfg, cinp, ginp, True)
    _, g2 = _run(cfg, cinp, ginp, True)
    for k in ("dx", "dw1", "dw3", "dw2", "d_topk_w"):
        assert torch.equal(g1[k], g2[k]), k


def test_training_step_full_size_sampled():
    """Mixtral-shaped forward + backward at full size; dX and d_topk_w on
    sampled tokens, dW1/dW3 rows and dW2 columns on sampled hidden units."""
    cfg = mi.MIXTRAL_TRAIN
    ginp = mi.make_inputs(cfg, 0, device=DEV, with_dy=True)
    desc = desc_of(cfg, save_acts=True)
    fb = L.alloc_forward(desc, DEV)
    L.forward(desc, ginp, fb)
    gb = L.alloc_backward(desc, DEV)
    L.backward(desc, ginp, fb, ginp["dy"], gb)
    torch.cuda.synchronize()
    idx, w, counts, *_ = check_routing_exact(cfg, {"logits_in": None, "bias": None,
                                                   "x": ginp["x"],
                                                   "wr": ginp["wr"]}, fb)
    g = torch.Generator().manual_seed(0)
    toks = sorted(set(torch.randint(0, cfg.T, (6,), generator=g).tolist()))
    cols = [(int(torch.randint(0, cfg.E, (1,), generator=g)),
             int(torch.randint(0, cfg.f, (1,), generator=g))) for _ in range(3)]
    ref = oracle.backward_sampled(ginp["x"], ginp["w1"], ginp["w3"],
                                  ginp["w2"], idx, w, ginp["dy"], toks, cols)
    t = torch.tensor(toks, device=DEV)
    assert rel_err(gb["dx"][t], ref["dx"]) <= 1e-2
    assert rel_err(gb["d_topk_w"][t], ref["d_w"]) <= 1e-2
    for i, (e, j) in enumerate(cols):
        assert rel_err(gb["dw1"][e, j], ref["dw1_rows"][i]) <= 1e-2, (e, j)
        assert rel_err(gb["dw3"][e, j], ref["dw3_rows"][i]) <= 1e-2, (e, j)
        assert rel_err(gb["dw2"][e, :, j], ref["dw2_cols"][i]) <= 1e-2, (e, j)
