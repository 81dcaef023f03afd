"""The grouped GEMMs' split of a partial last round of 256-row tiles into
128 x 128 quarter tiles (a second launch decided on the device from the
tile prefix).

The row-tile count is fixed by the offsets given to moe_grouped_gemm_swiglu:
17 tiles of 256 rows, so GEMM 1 (f / 128 = 16 column tiles) and GEMM 2
(d / 256 = 16) each have 272 tiles: one full round on 256 CUs and a last
round of 16, which is split. The last two experts make ragged tiles (255
and 1 rows), so some quarters are partial and some have no rows at all.
Split and unsplit results must be bit-identical (the same MFMA chain per
output), and sampled rows must match the fp64 oracle within the bf16
tolerance."""
import pytest
import torch

import oracle
from moe_testlib import DEV, rel_err
from ragged_grouped_gemm_router_amd import binding as B

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _run(desc, x_perm, offsets, routed, TK, d, f):
    h = torch.empty(TK, f, dtype=BF, device=DEV)
    y = torch.empty(TK, d, dtype=BF, device=DEV)
    ws = torch.empty(B.moe_workspace_size(desc), dtype=torch.uint8, device=DEV)
    B.moe_grouped_gemm_swiglu(desc, x_perm, None, offsets, routed, None, None,
                              h, y, None, None, None, ws)
    torch.cuda.synchronize()
    return h, y


def test_tail_split_bit_identical_and_matches_oracle():
    T, K, E, d, f = 2048, 2, 8, 4096, 2048
    counts = [512] * 6 + [511, 513]  # row tiles of 256: 6 * 2 + 2 + 3 = 17
    TK = T * K
    assert sum(counts) == TK
    off = [0]
    for c in counts:
        off.append(off[-1] + c)
    print(f"tail split: T{T} d{d} f{f} E{E} K{K} counts {counts}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(11)
    x_perm = torch.randn(TK, d, generator=g, device=DEV).to(BF)
    w1 = (torch.randn(E, f, d, generator=g, device=DEV) / d ** 0.5).to(BF)
    w3 = (torch.randn(E, f, d, generator=g, device=DEV) / d ** 0.5).to(BF)
    w2 = (torch.randn(E, d, f, generator=g, device=DEV) / f ** 0.5).to(BF)
    offsets = torch.tensor(off, dtype=torch.int32, device=DEV)
    routed = B.expert_weights(w1, w3, w2)

    desc = B.make_desc(T, d, f, E, K)
    h_split, y_split = _run(desc, x_perm, offsets, routed, TK, d, f)
    desc.flags = B.MOE_FLAG_NO_TAIL_SPLIT
    h_full, y_full = _run(desc, x_perm, offsets, routed, TK, d, f)
    assert torch.equal(h_split, h_full)
    assert torch.equal(y_split, y_full)

    # sampled rows: every expert's first and last row, plus rows of the
    # ragged tiles (expert 6's second tile, expert 7's one-row third tile)
    rows = sorted({r for e in range(E) for r in (off[e], off[e + 1] - 1)} |
                  {off[6] + 256, off[6] + 383, off[6] + 384, off[7] + 511,
                   off[7] + 512})
    offc = offsets.cpu()
    _, _, h_ref = oracle.stage_gemm1(x_perm.cpu(), offc, w1.cpu(), w3.cpu(),
                                     rows=rows)
    assert rel_err(h_split[rows].cpu(), h_ref) <= 1e-2
    y_ref = oracle.stage_gemm2(h_split.cpu(), offc, w2.cpu(), rows=rows)
    assert rel_err(y_split[rows].cpu(), y_ref) <= 1e-2



def test_tail_split_training_step_bit_identical():
    """Mixtral-shaped training step with and without the split: every
    output and gradient bit-identical. (With 8 experts of ~2048 rows the
    256-row tiles number 64-72; GEMM 2, 16 column tiles, splits its last
    round when that round holds at most 64 tiles.)"""
    from moe_testlib import desc_of, inputs
    from ragged_grouped_gemm_router_amd import layer as L
    import moe_inputs as mi
    cfg = mi.MIXTRAL_TRAIN
    _, ginp = inputs(cfg, seed=3, with_dy=True, device_gen=True)
    res = []
    for flags in (0, B.MOE_FLAG_NO_TAIL_SPLIT):
        desc = desc_of(cfg, save_acts=True)
        desc.flags |= flags
        fb = L.alloc_forward(desc, DEV)
        L.forward(desc, ginp, fb)
        gb = L.alloc_backward(desc, DEV)
        L.backward(desc, ginp, fb, ginp["dy"], gb)
        torch.cuda.synchronize()
        res.append((fb, gb))
    counts = res[0][0]["counts"].cpu()
    mt = int(((counts + 255) // 256).sum())
    S = torch.cuda.get_device_properties(0).multi_processor_count
    r = mt * 16 % S
    split = mt * 16 >= S and 0 < 4 * r <= S
    print(f"row tiles {mt}: last round {r} of GEMM 2's tiles "
          f"({'split' if split else 'not split'})", flush=True)
    (f0, g0), (f1, g1) = res
    for k in ("h", "y_perm", "out"):
        assert torch.equal(f0[k], f1[k]), k
    for k in ("dx", "dw1", "dw3", "dw2", "d_topk_w"):
        assert torch.equal(g0[k], g1[k]), k


def test_tail_split_mxfp8_training_step_bit_identical():
    """The same for the MXFP8 training step: its single-B products (GEMM 2
    and the backward's dx_perm product, 16 column tiles each) split their
    last round like the bf16 GEMM 2."""
    from moe_testlib import inputs
    from ragged_grouped_gemm_router_amd import layer as L
    import moe_inputs as mi
    cfg = mi.MIXTRAL_TRAIN
    _, ginp = inputs(cfg, seed=4, with_dy=True, device_gen=True)
    ginp = dict(ginp)
    ginp["mx"] = L.quantize_expert_weights(ginp)
    ginp["mx_bwd"] = L.quantize_expert_weights_bwd(ginp)
    res = []
    for flags in (0, B.MOE_FLAG_NO_TAIL_SPLIT):
        desc = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, cfg.f_shared,
                           gate=cfg.gate, mxfp8=True, save_acts=True)
        desc.flags |= flags
        fb = L.alloc_forward(desc, DEV)
        L.forward(desc, ginp, fb)
        gb = L.alloc_backward(desc, DEV)
        L.backward(desc, ginp, fb, ginp["dy"], gb)
        torch.cuda.synchronize()
        res.append((fb, gb))
    (f0, g0), (f1, g1) = res
    for k in ("y_perm", "out"):
        assert torch.equal(f0[k], f1[k]), k
    for k in ("dx", "dw1", "dw3", "dw2", "d_topk_w"):
        assert torch.equal(g0[k], g1[k]), k
