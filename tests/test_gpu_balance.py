"""Route-bias balance step and load monitor on the GPU against the oracle.
The bias step is a sign decision plus fp32 arithmetic that both sides do
in the same order: bit-exact. The monitor's min and cold count come from
the same fp32 window mean (exact); its entropy is within 1e-5."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import DEV, inputs, run_forward
from ragged_grouped_gemm_router_amd import binding as B

pytestmark = pytest.mark.gpu


def _step(desc, counts, bias, gamma, target, rule):
    b = torch.tensor(bias, dtype=torch.float32, device=DEV)
    load = torch.empty(desc.E, dtype=torch.float32, device=DEV)
    B.moe_update_route_bias(desc, torch.tensor(counts, dtype=torch.int32,
                                               device=DEV),
                            b, gamma, target, rule, load)
    torch.cuda.synchronize()
    return b.cpu().numpy(), load.cpu().numpy()


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("E", [2, 8, 256, 1024])
def test_bias_update_exact(E, rule):
    g = np.random.default_rng(E + rule)
    counts = g.integers(0, 500, E)
    counts[g.integers(0, E)] = 0
    bias = g.uniform(-0.1, 0.1, E).astype(np.float32)
    desc = B.make_desc(int(counts.sum()), 128, 128, E, 1)
    for target in (0.0, 1.5 / E):
        want_b, want_l = oracle.update_route_bias(bias, counts, 1e-3, target,
                                                  rule)
        got_b, got_l = _step(desc, counts, bias, 1e-3, target, rule)
        assert np.array_equal(got_l, want_l)
        assert np.array_equal(got_b, want_b)
    # balanced loads: unchanged
    even = np.full(E, 7)
    got_b, _ = _step(B.make_desc(7 * E, 128, 128, E, 1), even, bias, 1e-3,
                     0.0, rule)
    assert np.array_equal(got_b, bias)


def test_bias_update_after_forward():
    """The balance step on a DeepSeek-V3-like routing (sigmoid gate with a
    route bias), from the forward's own counts."""
    cfg = mi.MoEConfig("bal_T512_d256_f128_E64_K8", 512, 256, 128, 64, 8,
                       gate="sigmoid", bias=True)
    cinp, ginp = inputs(cfg, 3)
    desc, fb = run_forward(cfg, ginp)
    bias = cinp["bias"].numpy().astype(np.float32)
    b = torch.tensor(bias, device=DEV)
    B.moe_update_route_bias(desc, fb["counts"], b, 1e-3)
    torch.cuda.synchronize()
    want, _ = oracle.update_route_bias(bias, fb["counts"].cpu().numpy(), 1e-3)
    assert np.array_equal(b.cpu().numpy(), want)


@pytest.mark.parametrize("W,E", [(1, 8), (100, 256), (7, 1024), (3, 5)])
def test_balance_monitor(W, E):
    g = np.random.default_rng(W * E)
    hist = g.dirichlet(np.full(E, 0.5), W).astype(np.float32)
    out = torch.empty(3, dtype=torch.float32, device=DEV)
    B.moe_balance_monitor(B.make_desc(64, 128, 128, E, 1),
                          torch.tensor(hist, device=DEV), out)
    torch.cuda.synchronize()
    mn, ent, cold = oracle.balance_monitor(hist)
    o = out.cpu().numpy()
    assert o[0] == np.float32(mn)
    assert abs(float(o[1]) - ent) <= 1e-5 * max(abs(ent), 1.0)
    assert int(o[2]) == cold
