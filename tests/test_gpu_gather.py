"""Forward with gathered GEMM 1 rows (x_perm left out: the permute writes
only the indices and GEMM 1 reads row p from x[sorted_src[p] / K]).

The gathered forward is checked against the fp64 oracle (bf16 tolerance;
the fp8-aware oracle within 2e-2 under MXFP8) and, since it feeds GEMM 1
the same values in the same order, must equal the materialised forward
bit for bit."""
import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import DEV, check_routing_exact, desc_of, inputs, rel_err, tol
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

SMALL = [
    mi.MoEConfig("g_mixtral_like_T2048_d256_f512_E8_K2", 2048, 256, 512, 8, 2),
    mi.MoEConfig("g_deepseek_like_T256_d512_f256_E64_K8_shared", 256, 512,
                 256, 64, 8, f_shared=256, gate="sigmoid", bias=True),
    mi.MoEConfig("g_skewed_like_T2048_d256_f128_E32_K4", 2048, 256, 128, 32,
                 4, synth_logits=True, n_zero=4, zipf_s=1.2),
    mi.MoEConfig("g_tail_T333_d192_f256_E16_K3", 333, 192, 256, 16, 3),
    mi.MoEConfig("g_mid_rows_T1024_d256_f256_E16_K2", 1024, 256, 256, 16, 2),
]
MX_SMALL = [
    mi.MoEConfig("gmx_T1024_d256_f512_E8_K2", 1024, 256, 512, 8, 2),
    mi.MoEConfig("gmx_shared_sigmoid_T512_d256_f256_E16_K4_fs256", 512, 256,
                 256, 16, 4, f_shared=256, gate="sigmoid", bias=True),
]


def _both(desc, ginp):
    """The forward with x_perm materialised, then with gathered rows."""
    out = []
    for gather in (False, True):
        bufs = L.alloc_forward(desc, DEV, gather=gather)
        L.forward(desc, ginp, bufs)
        torch.cuda.synchronize()
        out.append(bufs)
    return out


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_gather_forward_parity(cfg):
    cinp, ginp = inputs(cfg, seed=4)
    mat, gat = _both(desc_of(cfg), ginp)
    idx, w, *_ = check_routing_exact(cfg, cinp, gat)
    ref = oracle.forward(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"], idx,
                         w, cinp["ws1"], cinp["ws3"], cinp["ws2"])
    assert rel_err(gat["out"], ref) <= tol(cfg)
    for k in ("sorted_src", "dest", "h", "y_perm", "out"):
        assert torch.equal(gat[k], mat[k]), k


@pytest.mark.parametrize("cfg", MX_SMALL, ids=[c.name for c in MX_SMALL])
def test_gather_mxfp8_forward_parity(cfg):
    cinp, ginp = inputs(cfg, seed=5)
    desc = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, cfg.f_shared,
                       gate=cfg.gate, mxfp8=True)
    ginp = dict(ginp)
    ginp["mx"] = L.quantize_expert_weights(ginp)
    mat, gat = _both(desc, ginp)
    idx, w, *_ = check_routing_exact(cfg, cinp, gat)
    ref = oracle.forward_mxfp8(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"],
                               idx, w, cinp["ws1"], cinp["ws3"], cinp["ws2"])
    assert rel_err(gat["out"], ref) <= 2e-2
    for k in ("h", "y_perm", "out"):
        assert torch.equal(gat[k], mat[k]), k


@pytest.mark.parametrize("cfg", [mi.MIXTRAL, mi.DEEPSEEK_V3],
                         ids=["mixtral", "deepseek_v3"])
def test_gather_forward_full_size(cfg):
    """Full sizes, in the benchmark's launch configuration: sampled tokens
    against the oracle, and the whole output against the materialised
    forward bit for bit."""
    ginp = mi.make_inputs(cfg, 0, device=DEV)
    mat, gat = _both(desc_of(cfg), ginp)
    small = {"logits_in": None, "x": ginp["x"], "wr": ginp["wr"],
             "bias": None if ginp["bias"] is None else ginp["bias"].cpu()}
    idx, w, *_ = check_routing_exact(cfg, small, gat)
    toks = [0, 1, cfg.T // 2, cfg.T - 1]
    ref = oracle.forward(ginp["x"], ginp["w1"], ginp["w3"], ginp["w2"], idx,
                         w, ginp["ws1"], ginp["ws3"], ginp["ws2"], tokens=toks)
    assert rel_err(gat["out"][torch.tensor(toks, device=DEV)], ref) <= 1e-2
    assert torch.equal(gat["out"], mat["out"])


def test_gather_needs_bf16_rows():
    cfg = mi.TINY_FP32
    desc = desc_of(cfg)
    _, ginp = inputs(cfg, seed=0)
    bufs = L.alloc_forward(desc, DEV, gather=True)
    with pytest.raises(B.MoeError) as ei:
        L.forward(desc, ginp, bufs)
    assert ei.value.status == B.MOE_EUNSUPPORTED
