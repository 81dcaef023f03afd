"""The allocation-free forward (moe_forward_noalloc, workspace in the
library's static device scratch) against the ordinary forward (caller's
workspace): same kernels in the same order, so every output must be
identical, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents)."""
import pytest
import torch

import moe_inputs as mi
from moe_testlib import DEV, desc_of, inputs
from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

pytestmark = pytest.mark.gpu

KEYS = ("logits", "topk_idx", "topk_w", "counts", "offsets", "sorted_src",
        "dest", "x_perm", "h", "y_perm", "y_shared", "out")


def _both(cfg, seed):
    _, ginp = inputs(cfg, seed=seed)
    desc = desc_of(cfg)
    assert B.moe_workspace_size(desc, False) <= B.MOE_STATIC_SCRATCH_BYTES
    ref = L.alloc_forward(desc, DEV)
    L.forward(desc, ginp, ref)
    got = L.alloc_forward(desc, DEV)
    L.forward_noalloc(desc, ginp, got)
    torch.cuda.synchronize()
    for k in KEYS:
        if ref.get(k) is None:
            continue
        assert torch.equal(got[k], ref[k]), (cfg.name, k)


def test_noalloc_forward_matches_forward_twice():
    big = mi.MoEConfig("qwen_like_T2048_d256_f192_E60_K4_fs384", 2048, 256,
                       192, 60, 4, f_shared=384)
    small = mi.MoEConfig("mixtral_like_T512_d128_f128_E8_K2", 512, 128, 128,
                         8, 2)
    _both(big, seed=7)
    _both(small, seed=8)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # a shared expert whose T x d_ff_shared bf16 hidden alone exceeds it
    cfg = mi.MoEConfig("too_big", 16384, 128, 128, 8, 2, f_shared=4096)
    desc = desc_of(cfg)
    assert B.moe_workspace_size(desc, False) > B.MOE_STATIC_SCRATCH_BYTES
    _, ginp = inputs(cfg.replace(T=8), seed=0)
    bufs = L.alloc_forward(desc_of(cfg.replace(T=8)), DEV)
    with pytest.raises(B.MoeError) as ei:
        L.forward_noalloc(desc, ginp, bufs)
    assert ei.value.status == B.MOE_EUNSUPPORTED
