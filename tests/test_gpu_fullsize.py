"""Parity at the full workload sizes, in the launch configuration the
benchmark times. Routing, counts, offsets and the permutation are checked
bit-exact over every token; outputs the oracle can compute one by one
(sampled tokens, sampled rows of h) are checked to the bf16 tolerance.
Inputs are drawn on the GPU (seeded) and read back by the oracle."""
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import DEV, check_routing_exact, rel_err, run_forward

pytestmark = pytest.mark.gpu

FULL = [mi.MIXTRAL, mi.DEEPSEEK_V3, mi.SKEWED, mi.QWEN_MOE]


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_full_size_forward_sampled(cfg):
    ginp = mi.make_inputs(cfg, 0, device=DEV)
    desc, bufs = run_forward(cfg, ginp, save_acts=False)
    small = {"x": ginp["x"], "wr": ginp["wr"],
             "logits_in": None if ginp["logits_in"] is None
             else ginp["logits_in"].cpu(),
             "bias": None if ginp["bias"] is None else ginp["bias"].cpu()}
    idx, w, counts, offsets, src, dest = check_routing_exact(cfg, small, bufs)
    if cfg.synth_logits:
        assert torch.equal(counts, ginp["loads"])
        assert int((counts == 0).sum()) >= 10
    else:
        std = bufs["logits"].float().std().item()
        assert 0.9 <= std <= 1.1, std
    g = torch.Generator().manual_seed(0)
    TK = cfg.TK
    rows = torch.randint(0, TK, (256,), generator=g)
    assert torch.equal(bufs["x_perm"][rows.to(DEV)].cpu(),
                       ginp["x"][(src[rows] // cfg.K).to(DEV)].cpu())
    # sampled rows of h and y_perm against the per-stage definitions
    hrows = torch.cat([torch.randint(0, TK, (6,), generator=g),
                       offsets[1:-1][counts[1:] > 0][:2] if cfg.E > 1 else
                       torch.zeros(0, dtype=torch.long), torch.tensor([TK - 1])])
    _, _, h = oracle.stage_gemm1(bufs["x_perm"], offsets, ginp["w1"],
                                 ginp["w3"], rows=hrows)
    assert rel_err(bufs["h"][hrows.to(DEV)], h) <= 1e-2
    y = oracle.stage_gemm2(bufs["h"], offsets, ginp["w2"], rows=hrows)
    assert rel_err(bufs["y_perm"][hrows.to(DEV)], y) <= 1e-2
    toks = sorted(set(torch.randint(0, cfg.T, (10,), generator=g).tolist()
                      + [0, cfg.T - 1]))
    ref = oracle.forward(ginp["x"], ginp["w1"], ginp["w3"], ginp["w2"], idx,
                         w, ginp["ws1"], ginp["ws3"], ginp["ws2"],
                         tokens=toks)
    err = rel_err(bufs["out"][torch.tensor(toks, device=DEV)], ref)
    assert err <= 1e-2, err
