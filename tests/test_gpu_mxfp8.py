"""MXFP8 path against the fp8-aware oracle: the quantiser and the quantised
permute bit-exact (codes and scales), the MXFP8 forward within 2e-2 of
max|ref| of the oracle that applies the same E8M0-scaled E4M3 rule; its
error against the exact (bf16-input) oracle is reported."""
import warnings

import pytest
import torch

import moe_inputs as mi
import oracle
from moe_testlib import DEV, check_routing_exact, inputs, rel_err
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

# Bound on the MXFP8 forward's error against the exact (bf16-input) layer,
# max|err| / max|ref|. E4M3 keeps 3 mantissa bits, so each MX-quantised
# element carries a relative rounding error of at most 2^-4, about uniform,
# rms 2^-4 / sqrt(3) = 0.036. A product of two quantised operands then has
# a relative error of rms about 0.051 per term, and with many independent
# terms the output error is about 0.051 of the output's rms. GEMM 2 adds
# the same again on top of GEMM 1's (h and W2 quantised): rms about 0.07
# of the output's rms, and the maxima of error and output over the sample
# are both a few times their rms, so max|err| / max|ref| lands near 0.07
# (measured: 0.067-0.084 on the small layers, 0.075 on the full-size
# Mixtral-shaped one). The bound is twice the largest relative rounding
# error of one E4M3 element, 2 * 2^-4.
MX_VS_EXACT = 0.125
F64 = torch.float64


def decode(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """E4M3 codes (uint8) times 2^(scale - 127) per 32 along the last dim."""
    v = codes.cpu().view(torch.float8_e4m3fn).to(F64)
    s = torch.pow(2.0, scales.cpu().to(F64) - 127.0)
    return (v.reshape(*v.shape[:-1], -1, 32) * s.unsqueeze(-1)).reshape(v.shape)


def special_matrix():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(48, 256, generator=g)
    x[0, :32] = 0.0                                   # all-zero block
    x[1, :32] *= 1e-30                                # tiny block
    x[2, :32] *= 1e30                                 # huge block
    x[3, :32] = 3.0                                   # exact (384 * 2^-7)
    x[4, 32:64] = torch.linspace(-500, 500, 32)       # saturating tail
    ladder = torch.tensor([1.0 + k / 16.0 for k in range(32)])
    x[5, :32] = ladder * 2.0 ** -3                    # E4M3 midpoints
    x[6] = x[6].sign() * torch.rand(256, generator=g) * 1e-3
    return x.to(torch.bfloat16)


def test_quantizer_bit_exact():
    x = special_matrix()
    q, s = L.quantize_mxfp8(x.to(DEV))
    torch.cuda.synchronize()
    ref_q, ref_c = oracle.mx_quantize(x.double())
    s = L.mx_scales_rows(s, x.shape[:-1])
    assert torch.equal(s.cpu(), ref_c)
    got = decode(q, s)
    want = oracle.mx_dequantize(ref_q, ref_c)
    assert torch.equal(got, want)   # -0.0 == 0.0 under equal()


MX_SMALL = [
    mi.MoEConfig("mx_T1024_d256_f512_E8_K2", 1024, 256, 512, 8, 2),
    mi.MoEConfig("mx_shared_sigmoid_T512_d256_f256_E16_K4_fs256", 512, 256,
                 256, 16, 4, f_shared=256, gate="sigmoid", bias=True),
    mi.MoEConfig("mx_T256_d128_f256_E8_K2", 256, 128, 256, 8, 2),
    mi.MoEConfig("mx_skewed_T1024_d256_f256_E16_K4", 1024, 256, 256, 16, 4,
                 synth_logits=True, n_zero=3, zipf_s=1.2),
]


def _mx_forward(cfg, ginp):
    desc = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, cfg.f_shared,
                       gate=cfg.gate, mxfp8=True)
    ginp = dict(ginp)
    ginp["mx"] = L.quantize_expert_weights(ginp)
    bufs = L.alloc_forward(desc, DEV)
    L.forward(desc, ginp, bufs)
    torch.cuda.synchronize()
    return desc, bufs, ginp["mx"]


@pytest.mark.parametrize("cfg", MX_SMALL, ids=[c.name for c in MX_SMALL])
def test_mxfp8_forward_parity(cfg):
    cinp, ginp = inputs(cfg, seed=3)
    desc, bufs, mx = _mx_forward(cfg, ginp)
    idx, w, counts, offsets, src, dest = check_routing_exact(cfg, cinp, bufs)
    # quantised permute: codes and scales of each x_perm row exact
    rq, rc = oracle.mx_quantize(cinp["x"][src // cfg.K].double())
    xs = L.mx_scales_rows(bufs["x_perm_scales"], (cfg.T * cfg.K,))
    assert torch.equal(xs.cpu(), rc)
    assert torch.equal(decode(bufs["x_perm"], xs), oracle.mx_dequantize(rq, rc))
    # weights quantised on the device agree with the oracle's rule (the
    # last expert: its rows come last in the stacked scale array)
    q1, c1 = oracle.mx_quantize(cinp["w1"][-1].double())
    w1s = L.mx_scales_rows(mx["w1_s"], (cfg.E, cfg.f))
    assert torch.equal(w1s[-1].cpu(), c1)
    sh = (cinp["ws1"], cinp["ws3"], cinp["ws2"])
    ref = oracle.forward_mxfp8(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"],
                               idx, w, *sh)
    err = rel_err(bufs["out"], ref)
    exact = oracle.forward(cinp["x"], cinp["w1"], cinp["w3"], cinp["w2"], idx, w,
                           *sh)
    err_exact = rel_err(bufs["out"], exact)
    warnings.warn(f"MXFP8 forward {cfg.name}: max|err|/max|ref| vs the "
                  f"fp8-aware oracle {err:.3e}, vs the bf16 (exact) oracle "
                  f"{err_exact:.3e}")
    assert err <= 2e-2, err
    assert err_exact <= MX_VS_EXACT, err_exact


def test_mxfp8_forward_full_size_sampled():
    """Mixtral-shaped MXFP8 forward; sampled tokens vs the fp8-aware
    oracle (which quantises the weights itself)."""
    cfg = mi.MIXTRAL_TRAIN
    ginp = mi.make_inputs(cfg, 0, device=DEV)
    desc, bufs, mx = _mx_forward(cfg, ginp)
    idx, w, *_ = check_routing_exact(cfg, {"logits_in": None, "bias": None,
                                      "x": ginp["x"], "wr": ginp["wr"]}, bufs)
    toks = [0, 17, 4095, cfg.T - 1]
    cache = {}
    ref = oracle.forward_mxfp8(ginp["x"], ginp["w1"], ginp["w3"], ginp["w2"],
                               idx, w, tokens=toks, weight_cache=cache)
    err = rel_err(bufs["out"][torch.tensor(toks, device=DEV)], ref)
    exact = oracle.forward(ginp["x"], ginp["w1"], ginp["w3"], ginp["w2"], idx,
                           w, tokens=toks)
    err_exact = rel_err(bufs["out"][torch.tensor(toks, device=DEV)], exact)
    warnings.warn(f"MXFP8 forward {cfg.name} (full size, tokens {toks}): "
                  f"max|err|/max|ref| vs the fp8-aware oracle {err:.3e}, vs "
                  f"the bf16 (exact) oracle {err_exact:.3e}")
    assert err <= 2e-2, err
    assert err_exact <= MX_VS_EXACT, err_exact
