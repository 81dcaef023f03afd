"""Pins of the CPU oracle against what the pages and the mathematics fix:
brute force on tiny inputs, closed forms, special cases that reduce to
library routines, invariants, and hand-worked examples. CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import moe_inputs as mi

F64 = torch.float64


def _rand_layer(T, d, f, E, K, seed=0, shared=0, gate="softmax", bias=False):
    cfg = mi.MoEConfig("t", T, d, f, E, K, f_shared=shared, gate=gate,
                       dtype="f32", bias=bias)
    inp = mi.make_inputs(cfg, seed)
    logits = inp["x"].float() @ inp["wr"].float().T
    idx, w = oracle.route(logits, K, gate, inp["bias"])
    return cfg, inp, logits, idx, w


# --------------------------------------------------------------- selection
def _subset_definition(keys_row, K):
    """The unique K-subset S such that every member beats every non-member
    under (key desc, id asc); found by trying every subset."""
    E = len(keys_row)
    wins = []
    for S in itertools.combinations(range(E), K):
        rest = [u for u in range(E) if u not in S]
        ok = all(keys_row[s] > keys_row[u] or
                 (keys_row[s] == keys_row[u] and s < u)
                 for s in S for u in rest)
        if ok:
            wins.append(S)
    assert len(wins) == 1
    return set(wins[0])


@pytest.mark.parametrize("E,K", [(1, 1), (3, 1), (5, 2), (6, 3), (7, 7), (7, 4)])
def test_topk_matches_subset_bruteforce(E, K):
    logits = torch.cat([mi.tie_logits(20, E),
                        torch.randn(20, E, generator=torch.Generator().manual_seed(E))])
    keys = oracle.selection_keys(logits)
    idx = oracle.topk_select(keys, K)
    for t in range(logits.shape[0]):
        row = keys[t].tolist()
        assert set(idx[t].tolist()) == _subset_definition(row, K)
        sel = idx[t].tolist()
        for a, b in zip(sel, sel[1:]):          # rank order of the K outputs
            assert row[a] > row[b] or (row[a] == row[b] and a < b)


def test_topk_with_bias_matches_bruteforce():
    g = torch.Generator().manual_seed(3)
    logits = torch.randn(30, 6, generator=g)
    bias = (torch.rand(6, generator=g) - 0.5) * 0.4
    keys = oracle.selection_keys(logits, bias)
    idx = oracle.topk_select(keys, 2)
    ref = (logits + bias).tolist()               # fp32 sums, as on the device
    for t in range(30):
        assert set(idx[t].tolist()) == _subset_definition(ref[t], 2)


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_all_equal_logits(gate):
    logits = torch.full((4, 8), 0.3)
    idx, w = oracle.route(logits, 3, gate)
    assert idx.tolist() == [[0, 1, 2]] * 4
    assert torch.allclose(w, torch.full((4, 3), 1 / 3, dtype=F64), rtol=0, atol=1e-15)


def test_k_equals_e_and_single_expert():
    logits = torch.tensor([[0.5, -1.0, 2.0, 0.5]])
    idx, w = oracle.route(logits, 4, "softmax")
    assert idx.tolist() == [[2, 0, 3, 1]]
    ref = torch.softmax(logits.double(), dim=1)[0, [2, 0, 3, 1]]
    assert torch.allclose(w[0], ref, rtol=1e-15, atol=0)
    idx, w = oracle.route(torch.tensor([[1.7], [-3.0]]), 1, "sigmoid")
    assert idx.tolist() == [[0], [0]] and w.tolist() == [[1.0], [1.0]]


def test_bias_flips_selection_but_not_weights():
    # selection on logits + bias, weights from raw sigmoid (P3 §6.3)
    logits = torch.tensor([[0.0, 0.05]])
    bias = torch.tensor([0.1, -0.1])
    idx, w = oracle.route(logits, 1, "sigmoid", bias)
    assert idx.tolist() == [[0]] and w.tolist() == [[1.0]]
    idx, w = oracle.route(logits, 2, "sigmoid", bias)
    assert idx.tolist() == [[0, 1]]
    s0, s1 = 1 / (1 + math.exp(-0.0)), 1 / (1 + math.exp(-float(np.float32(0.05))))
    assert abs(float(w[0, 0]) - s0 / (s0 + s1)) < 1e-15


def test_signed_zero_tie_and_nan():
    idx, _ = oracle.route(torch.tensor([[-0.0, 0.0], [0.0, -0.0]]), 1, "softmax")
    assert idx.tolist() == [[0], [0]]
    idx, _ = oracle.route(torch.tensor([[float("nan"), 1.0, -5.0]]), 2, "softmax")
    assert idx.tolist() == [[1, 2]]


def test_hand_worked_example():
    # logits [1, 2, 0], top-2: experts 2nd then 1st; softmax weights
    # e^2/(e^2+e) = e/(e+1) and 1/(e+1); sigmoid weights s(2)/(s(2)+s(1)).
    logits = torch.tensor([[1.0, 2.0, 0.0]])
    idx, w = oracle.route(logits, 2, "softmax")
    assert idx.tolist() == [[1, 0]]
    e = math.e
    assert abs(float(w[0, 0]) - e / (e + 1)) < 1e-15
    assert abs(float(w[0, 1]) - 1 / (e + 1)) < 1e-15
    idx, w = oracle.route(logits, 2, "sigmoid")
    s2, s1 = 1 / (1 + math.exp(-2)), 1 / (1 + math.exp(-1))
    assert abs(float(w[0, 0]) - s2 / (s1 + s2)) < 1e-15


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_weights_closed_forms(gate):
    g = torch.Generator().manual_seed(7)
    logits = torch.randn(64, 16, generator=g) * 3
    idx, w = oracle.route(logits, 4, gate)
    assert torch.allclose(w.sum(1), torch.ones(64, dtype=F64), rtol=0, atol=1e-12)
    L = logits.double()
    full = torch.softmax(L, 1) if gate == "softmax" else torch.sigmoid(L)
    sel = torch.gather(full, 1, idx)
    assert torch.allclose(w, sel / sel.sum(1, keepdim=True), rtol=1e-14, atol=0)


# ------------------------------------------------------------- permutation
def test_permutation_invariants_and_library_sort():
    cfg, inp, logits, idx, w = _rand_layer(97, 16, 8, 11, 3, seed=1)
    E, TK = 11, 97 * 3
    counts, offsets, src, dest = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert counts.tolist() == torch.bincount(flat, minlength=E).tolist()
    assert int(counts.sum()) == TK and int(offsets[-1]) == TK
    assert sorted(src.tolist()) == list(range(TK))
    assert (dest[src] == torch.arange(TK)).all()
    assert (src == torch.sort(flat, stable=True).indices).all()
    for e in range(E):
        grp = src[offsets[e]:offsets[e + 1]]
        assert (flat[grp] == e).all()
        assert (grp[1:] > grp[:-1]).all()


def test_zipf_synthesis_realises_designed_loads():
    T, E, K = 2048, 128, 8
    logits, loads = mi.synth_logits(T, E, K, 10, 1.2, 0)
    idx, w = oracle.route(logits, K, "softmax")
    counts, offsets, _, _ = oracle.permute(idx, E)
    assert counts.tolist() == loads.tolist()
    assert int((counts == 0).sum()) == 10 and int(counts.max()) <= T
    # at the full skewed shape the two largest experts hit the cap T
    full = mi.zipf_loads(16384, 128, 8, 10, 1.2, 0)
    assert sorted(full.tolist())[-2:] == [16384, 16384] and full.sum() == 131072


# ------------------------------------------------------------------ experts
def test_single_expert_is_textbook_swiglu():
    cfg, inp, logits, idx, w = _rand_layer(33, 24, 40, 1, 1, seed=2)
    out = oracle.forward(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w)
    x = inp["x"].double()
    ref = (F.silu(x @ inp["w1"][0].double().T) * (x @ inp["w3"][0].double().T)) \
        @ inp["w2"][0].double().T
    assert torch.allclose(out, ref, rtol=0, atol=1e-12 * ref.abs().max())


@pytest.mark.parametrize("shape", [(13, 8, 16, 5, 2, 0, "softmax"),
                                   (9, 16, 8, 6, 3, 12, "sigmoid"),
                                   (20, 8, 8, 7, 7, 0, "softmax")])
def test_three_formulations_agree(shape):
    T, d, f, E, K, fs, gate = shape
    cfg, inp, logits, idx, w = _rand_layer(T, d, f, E, K, seed=4, shared=fs, gate=gate)
    args = (inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w,
            inp["ws1"], inp["ws3"], inp["ws2"])
    a = oracle.forward(*args)
    b = oracle.forward_gather(*args)
    c = oracle.dense_masked_forward(*args)
    scale = a.abs().max()
    assert (a - b).abs().max() <= 1e-12 * scale
    assert (a - c).abs().max() <= 1e-12 * scale
    # token subsets give the same rows
    sub = [0, T // 2, T - 1]
    assert torch.equal(oracle.forward(*args, tokens=sub), a[sub]) or \
        (oracle.forward(*args, tokens=sub) - a[sub]).abs().max() <= 1e-13 * scale


def test_empty_expert_and_stage_composition():
    T, d, f, E, K = 16, 8, 12, 6, 2
    cfg, inp, logits, idx, w = _rand_layer(T, d, f, E, K, seed=5)
    idx = torch.where(idx == 3, torch.full_like(idx, 4), idx)  # expert 3 empty
    idx[:, 1] = torch.where(idx[:, 1] == idx[:, 0], (idx[:, 0] + 1) % E, idx[:, 1])
    idx = torch.where(idx == 3, torch.full_like(idx, 5), idx)
    assert (idx[:, 0] != idx[:, 1]).all() and not (idx == 3).any()
    counts, offsets, src, dest = oracle.permute(idx, E)
    assert counts[3] == 0
    x_perm = inp["x"][src // K]
    _, _, h = oracle.stage_gemm1(x_perm, offsets, inp["w1"], inp["w3"])
    y = oracle.stage_gemm2(h, offsets, inp["w2"])
    out = oracle.stage_combine(y, dest, w)
    ref = oracle.forward(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w)
    assert (out - ref).abs().max() <= 1e-12 * ref.abs().max()


def test_combine_k1_w1_is_inverse_permutation():
    T, d = 10, 4
    y = torch.randn(T, d).to(torch.bfloat16)
    dest = torch.randperm(T, generator=torch.Generator().manual_seed(0))
    out = oracle.stage_combine(y, dest, torch.ones(T, 1))
    assert torch.equal(out, y[dest].double())


# ----------------------------------------------------------------- backward
def _loss(inp, idx, w, dy, **over):
    args = dict(x=inp["x"], w1=inp["w1"], w3=inp["w3"], w2=inp["w2"])
    args.update(over)
    out = oracle.forward(args["x"], args["w1"], args["w3"], args["w2"], idx, w,
                         inp["ws1"], inp["ws3"], inp["ws2"])
    return float((out * dy.double()).sum())


@pytest.mark.parametrize("shared", [0, 6])
def test_backward_matches_finite_differences(shared):
    T, d, f, E, K = 7, 5, 6, 4, 2
    cfg, inp, logits, idx, w = _rand_layer(T, d, f, E, K, seed=6, shared=shared)
    for k in ("x", "w1", "w3", "w2", "ws1", "ws3", "ws2"):
        if inp[k] is not None:
            inp[k] = inp[k].double()
    dy = torch.randn(T, d, generator=torch.Generator().manual_seed(9), dtype=F64)
    g = oracle.backward(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w, dy,
                        inp["ws1"], inp["ws3"], inp["ws2"])
    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, key in [("x", "dx"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2")]:
        base = inp[name]
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in base.shape)
            p, m = base.clone(), base.clone()
            p[pos] += eps
            m[pos] -= eps
            fd = (_loss(inp, idx, w, dy, **{name: p}) -
                  _loss(inp, idx, w, dy, **{name: m})) / (2 * eps)
            assert abs(fd - float(g[key][pos])) <= 1e-6 * (1 + abs(fd)), (name, pos)
    for _ in range(4):
        t, k = int(rng.integers(0, T)), int(rng.integers(0, K))
        p, m = w.clone(), w.clone()
        p[t, k] += eps
        m[t, k] -= eps
        fd = (_loss(inp, idx, p, dy) - _loss(inp, idx, m, dy)) / (2 * eps)
        assert abs(fd - float(g["d_w"][t, k])) <= 1e-6 * (1 + abs(fd))
    if shared:
        for name, key in [("ws1", "dws1"), ("ws3", "dws3"), ("ws2", "dws2")]:
            base = inp[name]
            pos = tuple(int(rng.integers(0, s)) for s in base.shape)
            p, m = base.clone(), base.clone()
            p[pos] += eps
            m[pos] -= eps
            i2 = dict(inp)
            i2[name] = p
            lp = _loss(i2, idx, w, dy)
            i2[name] = m
            lm = _loss(i2, idx, w, dy)
            assert abs((lp - lm) / (2 * eps) - float(g[key][pos])) <= 1e-6


def test_backward_matches_autograd_dense():
    """Autograd through a dense masked layer built from library ops."""
    T, d, f, E, K = 9, 6, 10, 5, 2
    cfg, inp, logits, idx, w = _rand_layer(T, d, f, E, K, seed=8)
    x = inp["x"].double().requires_grad_()
    W1 = inp["w1"].double().requires_grad_()
    W3 = inp["w3"].double().requires_grad_()
    W2 = inp["w2"].double().requires_grad_()
    wl = w.clone().requires_grad_()
    G = torch.zeros(T, E, dtype=F64).scatter(1, idx, wl)
    h = F.silu(torch.einsum("td,efd->tef", x, W1)) * torch.einsum("td,efd->tef", x, W3)
    out = torch.einsum("tef,edf,te->td", h, W2, G)
    dy = torch.randn(T, d, generator=torch.Generator().manual_seed(1), dtype=F64)
    out.backward(dy)
    g = oracle.backward(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w, dy)
    for a, b in [(x.grad, g["dx"]), (W1.grad, g["dw1"]), (W3.grad, g["dw3"]),
                 (W2.grad, g["dw2"]), (wl.grad, g["d_w"])]:
        assert (a - b).abs().max() <= 1e-12 * (1 + b.abs().max())


def test_backward_sampled_equals_full():
    T, d, f, E, K = 24, 8, 16, 6, 2
    cfg, inp, logits, idx, w = _rand_layer(T, d, f, E, K, seed=10, shared=8)
    dy = torch.randn(T, d, generator=torch.Generator().manual_seed(2))
    args = (inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w, dy)
    sh = (inp["ws1"], inp["ws3"], inp["ws2"])
    full = oracle.backward(*args, *sh)
    toks = [0, 5, 23]
    cols = [(0, 0), (2, 7), (5, 15)]
    s = oracle.backward_sampled(*args, toks, cols, *sh)
    assert (s["dx"] - full["dx"][toks]).abs().max() <= 1e-12
    assert (s["d_w"] - full["d_w"][toks]).abs().max() <= 1e-12
    for i, (e, j) in enumerate(cols):
        assert (s["dw1_rows"][i] - full["dw1"][e, j]).abs().max() <= 1e-12
        assert (s["dw3_rows"][i] - full["dw3"][e, j]).abs().max() <= 1e-12
        assert (s["dw2_cols"][i] - full["dw2"][e, :, j]).abs().max() <= 1e-12


# -------------------------------------------------------------------- mxfp8
def test_e4m3_code_table():
    v = oracle.e4m3_values()
    fin = v[~torch.isnan(v)]
    assert fin.numel() == 254 and float(fin.max()) == 448.0
    assert float(fin[fin > 0].min()) == 2.0 ** -9
    assert torch.unique(fin).numel() == 253      # +0 and -0 coincide
    # the format's own table agrees with torch's e4m3fn decoding
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(F64)
    both_nan = torch.isnan(tv) & torch.isnan(v)
    assert (both_nan | (tv == v)).all()


def test_e4m3_round_identity_ties_and_library_cast():
    v = oracle.e4m3_values()
    fin = v[~torch.isnan(v)]
    assert torch.equal(oracle.e4m3_round(fin), fin)
    # midpoints between neighbours go to the even mantissa
    assert float(oracle.e4m3_round(torch.tensor([1.0625]))) == 1.0
    assert float(oracle.e4m3_round(torch.tensor([1.1875]))) == 1.25
    assert float(oracle.e4m3_round(torch.tensor([500.0]))) == 448.0
    assert float(oracle.e4m3_round(torch.tensor([-464.0]))) == -448.0
    # against the library cast (RNE, non-saturating) after clamping to 448
    g = torch.Generator().manual_seed(0)
    r = torch.cat([torch.randn(20000, generator=g, dtype=F64) * s
                   for s in (1e-3, 0.1, 1, 30, 300)])
    mids = ((torch.sort(torch.unique(fin)).values[1:] +
             torch.sort(torch.unique(fin)).values[:-1]) / 2)
    r = torch.cat([r, mids, -mids])
    lib = r.clamp(-448, 448).to(torch.float8_e4m3fn).to(F64)
    assert torch.equal(oracle.e4m3_round(r).abs(), lib.abs())


def test_mx_block_rule():
    # amax 3 -> X = floor(log2 3) - 8 = -7, 3 * 2^7 = 384 is exact in E4M3
    v = torch.full((1, 32), 3.0, dtype=F64)
    q, c = oracle.mx_quantize(v)
    assert int(c[0, 0]) == 127 - 7 and torch.equal(q, torch.full_like(v, 384.0))
    assert torch.equal(oracle.mx_dequantize(q, c), v)
    # an all-zero block gets scale code 0 and zero elements
    q, c = oracle.mx_quantize(torch.zeros(2, 64, dtype=F64))
    assert c.tolist() == [[0, 0], [0, 0]] and (q == 0).all()
    # blocks made of E4M3 values times a power of two quantise exactly
    vals = oracle.e4m3_values()
    fin = vals[~torch.isnan(vals)]
    g = torch.Generator().manual_seed(1)
    for X in (-20, -3, 0, 5):
        blk = fin[torch.randint(0, fin.numel(), (4, 32), generator=g)]
        blk[:, 0] = 448.0                        # amax in [256, 512)
        v = blk * 2.0 ** X
        q, c = oracle.mx_quantize(v)
        assert (c == 127 + X).all()
        assert torch.equal(oracle.mx_dequantize(q, c), v)
    # error bound of one quantisation: with X = floor(log2 amax) - 8 the
    # scaled block max lies in [256, 512); elements whose scaled value is at
    # most 448 round with error <= |v| 2^-4 (normal) or 2^(X-10)
    # (subnormal); larger ones saturate to 448 * 2^X, an error below amax/8
    v = torch.randn(64, 256, generator=g, dtype=F64)
    rt = oracle.mx_roundtrip(v).reshape(64, 8, 32)
    blocks = v.reshape(64, 8, 32)
    amax = blocks.abs().amax(-1, keepdim=True)
    _, ex = torch.frexp(amax)
    scale = torch.pow(2.0, ex.double() - 1 - 8)
    err = (rt - blocks).abs()
    inrange = blocks.abs() <= 448 * scale
    assert (err[inrange] <= (blocks.abs() * 2.0 ** -4 + scale * 2.0 ** -10)[inrange]).all()
    assert (err[~inrange] == (blocks.abs() - 448 * scale)[~inrange]).all()
    assert (err <= amax / 8).all() and (~inrange).any()


def test_mxfp8_forward_close_to_exact():
    cfg, inp, logits, idx, w = _rand_layer(40, 64, 96, 4, 2, seed=11)
    exact = oracle.forward(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w)
    q = oracle.forward_mxfp8(inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w)
    rel = (q - exact).abs().max() / exact.abs().max()
    assert 1e-4 < float(rel) < 0.2


# --------------------------------------------------------------- accounting
def test_accounting_against_page_figures():
    import json
    import os
    from ragged_grouped_gemm_router_amd import accounting as acc
    p = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
    g = json.load(open(p))
    c = g["comm_bytes_per_token_layer"]
    b = acc.comm_bytes_per_token(c["K"], c["D"], c["bytes_per_elem"])
    assert round(b / 1000) == c["printed_kB"]
    v = g["v3_training_flops"]
    fl = acc.training_flops_6nt(v["N_act"], v["T"])
    assert abs(fl / v["printed"] - 1) < 0.01
    h = g["v3_gpu_hours"]
    hours = h["flops"] / (h["effective_tflops"] * 1e12 * 3600)
    assert abs(hours / h["printed_hours"] - 1) < 0.01
    a = g["v3_active_fraction"]
    assert round(100 * a["active"] / a["total"], 1) == a["printed_pct"]
    cb = g["fine_grained_combinations"]
    assert math.comb(8, 2) == cb["n8_k2_printed"]
    # the printed ~4e11 for C(256, 8) is wrong by 10^3 (it is ~4.1e14): not a pin
    assert 4.0e14 < math.comb(256, 8) < 4.2e14
    # a SwiGLU expert is three d x f matrices, so 6 d f flops per copy
    assert acc.routed_fwd_flops(4096, 14336, 16384) == 5_772_436_045_824
    assert acc.train_flops(acc.routed_fwd_flops(1, 1, 1)) == 18


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_router_backward_matches_autograd(gate):
    """The closed-form gate Jacobian equals autograd through
    logits = x Wr^T, a fixed selection and the renormalised weights."""
    g = torch.Generator().manual_seed(11)
    T, d, E, K = 12, 10, 6, 3
    x = torch.randn(T, d, generator=g, dtype=torch.float64)
    wr = torch.randn(E, d, generator=g, dtype=torch.float64)
    d_w = torch.randn(T, K, generator=g, dtype=torch.float64)
    idx = oracle.topk_select(oracle.selection_keys(x @ wr.T), K)
    xa, wra = x.clone().requires_grad_(), wr.clone().requires_grad_()
    L = xa @ wra.T
    Ls = torch.gather(L, 1, idx)
    z = torch.softmax(Ls, dim=1) if gate == "softmax" else torch.sigmoid(Ls)
    wt = z / z.sum(dim=1, keepdim=True)
    (wt * d_w).sum().backward()
    L0 = (x @ wr.T).detach()
    w = oracle.gate_weights(L0, idx, gate)
    r = oracle.router_backward(x, wr, L0, idx, w, d_w, gate)
    assert torch.allclose(r["d_wr"], wra.grad, rtol=0, atol=1e-12)
    assert torch.allclose(r["dx"], xa.grad, rtol=0, atol=1e-12)
    # unselected logits get exactly zero
    mask = torch.zeros(T, E, dtype=torch.bool)
    mask.scatter_(1, idx, True)
    assert torch.all(r["d_logits"][~mask] == 0)


def test_router_backward_invariants():
    """softmax: the logit gradient of a token sums to zero (shifting all
    logits leaves the weights unchanged); uniform d_w gives zero gradient
    in both modes (the weights always sum to one)."""
    g = torch.Generator().manual_seed(12)
    T, E, K = 9, 8, 4
    L = torch.randn(T, E, generator=g, dtype=torch.float64)
    idx = oracle.topk_select(oracle.selection_keys(L), K)
    d_w = torch.randn(T, K, generator=g, dtype=torch.float64)
    w = oracle.gate_weights(L, idx, "softmax")
    dl = oracle.gate_logit_grad(L, idx, w, d_w, "softmax")
    assert torch.allclose(dl.sum(dim=1), torch.zeros(T, dtype=torch.float64),
                          atol=1e-14)
    for gate in ("softmax", "sigmoid"):
        w = oracle.gate_weights(L, idx, gate)
        dl = oracle.gate_logit_grad(L, idx, w, torch.full((T, K), 0.7,
                                    dtype=torch.float64), gate)
        assert torch.allclose(dl, torch.zeros_like(dl), atol=1e-14)


# --------------------------------------------------------------------------
# Load-balance statistics [P3 §6.2, §9]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_balance_stats_closed_forms(gate):
    """Uniform logits give P_i = 1/E for any routing, so aux = sum_i f_i =
    K; top-1 routing spread evenly with uniform probabilities gives aux = 1,
    the value the page scales the loss by E to reach [P3 §6.2]."""
    T, E, K = 24, 6, 2
    L = torch.zeros(T, E, dtype=torch.float64)
    g = torch.Generator().manual_seed(21)
    idx = torch.stack([torch.randperm(E, generator=g)[:K] for _ in range(T)])
    r = oracle.load_balance_stats(L, idx, E, gate)
    assert torch.allclose(r["p_mean"], torch.full((E,), 1.0 / E,
                          dtype=torch.float64), atol=1e-15)
    assert abs(float(r["aux"]) - K) < 1e-12
    idx1 = (torch.arange(T) % E).unsqueeze(1)
    r1 = oracle.load_balance_stats(L, idx1, E, gate)
    assert torch.allclose(r1["f"], torch.full((E,), 1.0 / E,
                          dtype=torch.float64), atol=1e-15)
    assert abs(float(r1["aux"]) - 1.0) < 1e-12


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_balance_stats_invariants(gate):
    """f equals bincount / T and sums to K; each token's probabilities sum
    to one, so p_mean sums to one; evenly spread loads (every f_i = K/E)
    make aux = K whatever the logits."""
    g = torch.Generator().manual_seed(22)
    T, E, K = 40, 8, 3
    L = 2.0 * torch.randn(T, E, generator=g, dtype=torch.float64)
    idx = oracle.topk_select(oracle.selection_keys(L), K)
    r = oracle.load_balance_stats(L, idx, E, gate)
    assert torch.equal(r["f"], torch.bincount(idx.reshape(-1), minlength=E)
                       .to(torch.float64) / T)
    assert abs(float(r["f"].sum()) - K) < 1e-12
    assert abs(float(r["p_mean"].sum()) - 1.0) < 1e-12
    # every token picks experts (t + j) mod E: each expert T*K/E times
    idx_even = (torch.arange(T).unsqueeze(1) + torch.arange(K)) % E
    r2 = oracle.load_balance_stats(L, idx_even, E, gate)
    assert abs(float(r2["aux"]) - K) < 1e-12


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_aux_loss_grad_matches_autograd(gate):
    """The closed-form logit gradient of the balance loss equals autograd
    through softmax (or the normalised sigmoid) and the token mean, with
    the mask share held fixed; added into the router backward it reaches
    Wr and x as aux_coef times autograd of the balance loss."""
    g = torch.Generator().manual_seed(23)
    T, d, E, K = 14, 9, 7, 2
    x = torch.randn(T, d, generator=g, dtype=torch.float64)
    wr = torch.randn(E, d, generator=g, dtype=torch.float64)
    L0 = x @ wr.T
    idx = oracle.topk_select(oracle.selection_keys(L0), K)
    f = torch.bincount(idx.reshape(-1), minlength=E).to(torch.float64) / T
    xa, wra = x.clone().requires_grad_(), wr.clone().requires_grad_()
    La = xa @ wra.T
    if gate == "softmax":
        P = torch.softmax(La, dim=1)
    else:
        s = torch.sigmoid(La)
        P = s / s.sum(dim=1, keepdim=True)
    aux = E * (f * P.mean(dim=0)).sum()
    coef = 0.03
    (coef * aux).backward()
    dl = oracle.aux_loss_logit_grad(L0, idx, E, gate)
    zero = torch.zeros(T, K, dtype=torch.float64)
    w = oracle.gate_weights(L0, idx, gate)
    r = oracle.router_backward(x, wr, L0, idx, w, zero, gate, aux_coef=coef)
    assert torch.allclose(r["d_logits"], coef * dl, rtol=0, atol=1e-15)
    assert torch.allclose(r["d_wr"], wra.grad, rtol=0, atol=1e-12)
    assert torch.allclose(r["dx"], xa.grad, rtol=0, atol=1e-12)


def test_aux_loss_grad_special_cases():
    """Softmax: a token's gradient sums to zero (shift invariance); evenly
    spread loads give zero gradient (aux is then K for every logit)."""
    g = torch.Generator().manual_seed(24)
    T, E, K = 16, 8, 2
    L = torch.randn(T, E, generator=g, dtype=torch.float64)
    idx = oracle.topk_select(oracle.selection_keys(L), K)
    dl = oracle.aux_loss_logit_grad(L, idx, E, "softmax")
    assert torch.allclose(dl.sum(dim=1), torch.zeros(T, dtype=torch.float64),
                          atol=1e-15)
    assert dl.abs().max() > 1e-3
    idx_even = (torch.arange(T).unsqueeze(1) + torch.arange(K)) % E
    for gate in ("softmax", "sigmoid"):
        dz = oracle.aux_loss_logit_grad(L, idx_even, E, gate)
        assert dz.abs().max() < 1e-15


# --------------------------------------------------------------------------
# Bias-balance update and load monitor [P3 §6.3, §9, §13.9]
# --------------------------------------------------------------------------

def test_route_bias_update_page_rule():
    """The stated rule: overloaded experts' bias drops by gamma,
    underloaded ones' rises by gamma; the scaled variant moves each by
    gamma times its load. Two experts at 3:1 against the 1/2 target."""
    bias = np.array([0.25, -0.5], dtype=np.float32)
    nb, load = oracle.update_route_bias(bias, [300, 100], 0.125)
    assert load.tolist() == [0.75, 0.25]
    assert nb.tolist() == [0.125, -0.375]
    nb1, _ = oracle.update_route_bias(bias, [300, 100], 0.125, rule=1)
    assert nb1.tolist() == [0.25 - 0.125 * 0.75, -0.5 + 0.125 * 0.25]


def test_route_bias_update_invariants():
    """Balanced loads leave the bias unchanged; an explicit target moves
    experts on either side of it; an empty expert's scaled step uses the
    1e-6 floor; the plain rule's steps sum to gamma * (#under - #over)."""
    E = 8
    bias = np.linspace(-1, 1, E).astype(np.float32)
    nb, _ = oracle.update_route_bias(bias, [64] * E, 0.01)
    assert np.array_equal(nb, bias)
    counts = [0, 5, 10, 10, 10, 10, 20, 15]
    nb, load = oracle.update_route_bias(bias, counts, 0.01, target=0.1)
    assert np.array_equal(np.sign(bias - nb), np.sign(load - np.float32(0.1)))
    nb1, _ = oracle.update_route_bias(bias, counts, 0.5, rule=1)
    assert nb1[0] == np.float32(bias[0] - np.float32(-0.5) * np.float32(1e-6))
    nb0, _ = oracle.update_route_bias(np.zeros(E, np.float32), counts, 0.5)
    n_under = sum(c / 80 < 1 / E for c in counts)
    n_over = sum(c / 80 > 1 / E for c in counts)
    assert abs(float(nb0.sum()) - 0.5 * (n_under - n_over)) < 1e-6


def test_balance_monitor_closed_forms():
    """Uniform loads: min 1/E, entropy log E (up to the 1e-9 guard), no
    cold expert. All load on one expert: entropy ~0, E - 1 cold experts.
    A window averages its rows."""
    E = 16
    mn, ent, cold = oracle.balance_monitor(np.full((5, E), 1.0 / E))
    assert abs(mn - 1.0 / E) < 1e-8
    assert abs(ent - math.log(E)) < 1e-6
    assert cold == 0
    one = np.zeros((3, E))
    one[:, 3] = 1.0
    mn, ent, cold = oracle.balance_monitor(one)
    assert mn == 0.0 and abs(ent) < 1e-8 and cold == E - 1
    # two rows that average to uniform
    a = np.zeros((2, E))
    a[0, : E // 2] = 2.0 / E
    a[1, E // 2:] = 2.0 / E
    mn, ent, cold = oracle.balance_monitor(a)
    assert abs(mn - 1.0 / E) < 1e-8 and cold == 0


# --------------------------------------------------------------------------
# MXFP8 backward [P3 §13.6]
# --------------------------------------------------------------------------

def _mx_bwd_case(seed, T=40, d=64, f=96, E=4, K=2):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, d, generator=g, dtype=torch.float64)
    w1 = torch.randn(E, f, d, generator=g, dtype=torch.float64) / d ** 0.5
    w3 = torch.randn(E, f, d, generator=g, dtype=torch.float64) / d ** 0.5
    w2 = torch.randn(E, d, f, generator=g, dtype=torch.float64) / f ** 0.5
    L = torch.randn(T, E, generator=g, dtype=torch.float64)
    idx = oracle.topk_select(oracle.selection_keys(L), K)
    idx[0] = torch.arange(K)  # expert 3 may stay empty
    w = oracle.gate_weights(L, idx, "softmax")
    dy = torch.randn(T, d, generator=g, dtype=torch.float64)
    return x, w1, w3, w2, idx, w, dy


def test_mx_backward_without_quantisers_is_exact():
    """With every quantiser (and the bf16 storage rounding) the identity,
    the MXFP8 backward is the exact backward: which operand meets which,
    signs and the SwiGLU derivative are those of the layer."""
    x, w1, w3, w2, idx, w, dy = _mx_bwd_case(31)
    got = oracle.backward_mxfp8(x, w1, w3, w2, idx, w, dy, quant=False)
    ref = oracle.backward(x, w1, w3, w2, idx, w, dy)
    for k in ("dx", "dw1", "dw3", "dw2", "d_w"):
        assert torch.allclose(got[k], ref[k], rtol=0, atol=1e-12), k


def test_mx_cols_quantiser_axis():
    """A transposed operand is quantised in blocks along its first
    dimension: a matrix whose 32-blocks down each column are exactly
    representable (integers of magnitude <= 14 times a power of two per
    column, so at most 448 after scaling) is left unchanged, while
    quantising along rows, which mixes the columns' scales 2^0..2^20 and
    so drops the small ones below E4M3's subnormal step, is not."""
    g = torch.Generator().manual_seed(32)
    ints = torch.randint(-14, 15, (64, 32), generator=g).to(torch.float64)
    col_scale = torch.pow(2.0, torch.arange(32, dtype=torch.float64) % 21)
    W = ints * col_scale
    assert torch.equal(oracle.mx_roundtrip_cols(W), W)
    assert not torch.equal(oracle.mx_roundtrip(W), W)


def test_mx_backward_sampled_matches_full_and_is_near_exact():
    """The sampled form reproduces the full MXFP8 backward on its sample,
    and the MXFP8 gradients stay near the exact ones (a sanity bound: E4M3
    keeps 3 mantissa bits, and these experts have few rows)."""
    x, w1, w3, w2, idx, w, dy = _mx_bwd_case(33)
    full = oracle.backward_mxfp8(x, w1, w3, w2, idx, w, dy)
    toks = [0, 5, 39]
    cols = [(0, 0), (1, 37), (2, 95)]
    smp = oracle.backward_mxfp8_sampled(x, w1, w3, w2, idx, w, dy, toks, cols)
    assert torch.allclose(smp["dx"], full["dx"][toks], rtol=0, atol=1e-12)
    assert torch.allclose(smp["d_w"], full["d_w"][toks], rtol=0, atol=1e-12)
    for i, (e, j) in enumerate(cols):
        assert torch.allclose(smp["dw1_rows"][i], full["dw1"][e, j], atol=1e-12)
        assert torch.allclose(smp["dw3_rows"][i], full["dw3"][e, j], atol=1e-12)
        assert torch.allclose(smp["dw2_cols"][i], full["dw2"][e, :, j], atol=1e-12)
    exact = oracle.backward(x, w1, w3, w2, idx, w, dy)
    for k in ("dx", "dw1", "dw3", "dw2", "d_w"):
        err = (full[k] - exact[k]).abs().max() / exact[k].abs().max()
        assert 0 < err < 0.3, (k, float(err))


def test_mx_backward_shared_expert_reduces():
    """With identity quantisers the shared expert's MXFP8 backward is the
    exact shared-expert backward; a zero shared expert adds nothing."""
    x, w1, w3, w2, idx, w, dy = _mx_bwd_case(34, f=64)
    g = torch.Generator().manual_seed(35)
    d, fs = x.shape[1], 96
    ws1 = torch.randn(fs, d, generator=g, dtype=torch.float64) / d ** 0.5
    ws3 = torch.randn(fs, d, generator=g, dtype=torch.float64) / d ** 0.5
    ws2 = torch.randn(d, fs, generator=g, dtype=torch.float64) / fs ** 0.5
    got = oracle.backward_mxfp8(x, w1, w3, w2, idx, w, dy, ws1, ws3, ws2,
                                quant=False)
    ref = oracle.backward(x, w1, w3, w2, idx, w, dy, ws1, ws3, ws2)
    for k in ("dx", "dw1", "dw3", "dw2", "d_w", "dws1", "dws3", "dws2"):
        assert torch.allclose(got[k], ref[k], rtol=0, atol=1e-12), k
    z = torch.zeros_like
    with_zero = oracle.backward_mxfp8(x, w1, w3, w2, idx, w, dy, z(ws1),
                                      z(ws3), z(ws2))
    without = oracle.backward_mxfp8(x, w1, w3, w2, idx, w, dy)
    assert torch.equal(with_zero["dx"], without["dx"])


# --------------------------------------------------------------------------
# MXFP8 forward: which operand is blocked along which axis [P2, section on
# the TE mechanisms: MXFP8 grouped GEMM operands; P3 §13.6 per-tile scales]
# --------------------------------------------------------------------------

def test_mxfp8_forward_without_quantisers_is_exact():
    """With every quantiser the identity the MXFP8 forward is the exact
    layer, shared expert included: no other arithmetic differs."""
    cfg, inp, logits, idx, w = _rand_layer(24, 64, 96, 4, 2, seed=41, shared=64)
    args = (inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w,
            inp["ws1"], inp["ws3"], inp["ws2"])
    got = oracle.forward_mxfp8(*args, quant=False)
    ref = oracle.forward(*args)
    assert (got - ref).abs().max() <= 1e-12 * ref.abs().max()


def _mx_exact_rows(rows, cols, scale_of_row, g):
    """A matrix whose 32-blocks along each row are exactly representable
    in MX (E4M3 values times 2^X, each block's largest magnitude 448 so
    that X = floor(log2 amax) - 8 is the X used), with row r scaled by
    scale_of_row(r). Rows with different scales make the 32-blocks down a
    column mix magnitudes 2^8 apart and more, which E4M3's 3 mantissa bits
    and subnormal floor cannot hold: those blocks are not exact."""
    vals = oracle.e4m3_values()
    fin = vals[~torch.isnan(vals)]
    m = fin[torch.randint(0, fin.numel(), (rows, cols), generator=g)]
    m.view(rows, cols // 32, 32)[:, :, 0] = 448.0 * torch.where(
        torch.rand(rows, cols // 32, generator=g) < 0.5, -1.0, 1.0).to(F64)
    s = torch.tensor([float(scale_of_row(r)) for r in range(rows)], dtype=F64)
    return m * s.unsqueeze(1)


def test_mxfp8_forward_quantiser_axes():
    """Inputs exact in 32-blocks along each GEMM's contraction axis (x and
    W1/W3 along d_model, W2 along d_ff) and not along the other axis: the
    MXFP8 forward must then equal the exact GEMM 1, h MX-rounded along
    d_ff, the exact GEMM 2 and the combine, composed from the stage
    functions (to rounding). An oracle that left h unquantised, or blocked
    x, W1/W3 or W2 along their other axis, differs by far more; the test
    shows that too, so the construction discriminates."""
    g = torch.Generator().manual_seed(42)
    T, d, f, E, K = 64, 64, 96, 3, 2
    x = _mx_exact_rows(T, d, lambda r: 2.0 ** (r % 9 - 12), g)
    w1 = torch.stack([_mx_exact_rows(f, d, lambda r: 2.0 ** (-(r % 11) - 10), g)
                      for _ in range(E)])
    w3 = torch.stack([_mx_exact_rows(f, d, lambda r: 2.0 ** (-(r % 7) - 10), g)
                      for _ in range(E)])
    w2 = torch.stack([_mx_exact_rows(d, f, lambda r: 2.0 ** (-(r % 10) - 10), g)
                      for _ in range(E)])
    assert torch.equal(oracle.mx_roundtrip(x), x)
    for W in (w1, w3, w2):
        assert torch.equal(oracle.mx_roundtrip(W), W)
        assert not torch.equal(oracle.mx_roundtrip_cols(W[0]), W[0])
    assert not torch.equal(oracle.mx_roundtrip(x.T).T, x)
    L = torch.randn(T, E, generator=g, dtype=F64).float()
    idx, w = oracle.route(L, K, "softmax")
    counts, offsets, src, dest = oracle.permute(idx, E)
    assert (counts > 0).all()

    def composed(xx, W1, W3, W2, hq=oracle.mx_roundtrip):
        _, _, h = oracle.stage_gemm1(xx[src // K], offsets, W1, W3)
        return oracle.stage_combine(oracle.stage_gemm2(hq(h), offsets, W2),
                                    dest, w)

    got = oracle.forward_mxfp8(x, w1, w3, w2, idx, w)
    ref = composed(x, w1, w3, w2)
    scale = ref.abs().max()
    assert (got - ref).abs().max() <= 1e-12 * scale
    cols = lambda W: torch.stack([oracle.mx_roundtrip_cols(m) for m in W])  # noqa: E731
    wrong = {
        "h unquantised": composed(x, w1, w3, w2, hq=lambda h: h),
        "h along tokens": composed(x, w1, w3, w2,
                                   hq=lambda h: oracle.mx_roundtrip_cols(h)),
        "x along tokens": composed(oracle.mx_roundtrip(x.T).T, w1, w3, w2),
        "W1 along d_ff": composed(x, cols(w1), w3, w2),
        "W3 along d_ff": composed(x, w1, cols(w3), w2),
        "W2 along d_model": composed(x, w1, w3, cols(w2)),
    }
    for name, v in wrong.items():
        assert (v - ref).abs().max() > 1e-6 * scale, name


def test_mx_backward_quantiser_placement():
    """Which quantiser meets which operand in the MXFP8 backward of one
    expert: identity quantisers that record what they are applied to show
    the data-gradient products take W2, W1 and W3 through the column
    quantiser (blocks along their first dimension: d_model for W2 [d, f],
    d_ff for W1, W3 [f, d], the contraction of dh = g W2 and of
    dx = da W1 + db W3), and that the forward's weights, its h, the output
    gradient g and da, db go through the row quantiser (blocks along their
    last dimension). With the column quantiser's axis pinned separately,
    this fixes every block axis of the backward."""
    from oracle import mxfp8 as M
    g = torch.Generator().manual_seed(43)
    n, d, f = 20, 64, 96
    X = torch.randn(n, d, generator=g, dtype=F64)
    W1 = torch.randn(f, d, generator=g, dtype=F64)
    W3 = torch.randn(f, d, generator=g, dtype=F64)
    W2 = torch.randn(d, f, generator=g, dtype=F64)
    G = torch.randn(n, d, generator=g, dtype=F64)
    rows, colq = [], []

    def Q(v):
        rows.append(v.clone())
        return v

    def Qc(v):
        colq.append(v.clone())
        return v

    dX, dW1, dW3, dW2, Y = M._mx_ffn_bwd(X, W1, W3, W2, G, Q, Qc, lambda v: v)

    def count(lst, t):
        return sum(1 for v in lst if v.shape == t.shape and torch.equal(v, t))

    for W in (W1, W3, W2):
        assert count(colq, W) == 1 and count(rows, W) == 1
    assert len(colq) == 3
    assert count(rows, G) == 1
    a, b = X @ W1.T, X @ W3.T
    h = oracle.swiglu(a, b)
    assert count(rows, h) == 1
    # da and db are the row-quantised [n, f] operands other than h
    others = [v for v in rows if v.shape == (n, f) and not torch.equal(v, h)]
    assert len(others) == 2 and len(rows) == 7
    ref = oracle.backward(X, W1.unsqueeze(0), W3.unsqueeze(0), W2.unsqueeze(0),
                          torch.zeros(n, 1, dtype=torch.long),
                          torch.ones(n, 1, dtype=F64), G)
    assert torch.allclose(dX, ref["dx"], rtol=0, atol=1e-10)
    assert torch.allclose(dW1, ref["dw1"][0], rtol=0, atol=1e-10)
    assert torch.allclose(dW2, ref["dw2"][0], rtol=0, atol=1e-10)


def test_backward_gradcheck():
    """torch.autograd.gradcheck on the oracle's closed-form backward: a
    function whose forward is oracle.forward and whose backward is
    oracle.backward must agree with central finite differences of the
    forward in every input (x, W1, W3, W2, the gate weights, shared
    expert weights), routing fixed."""
    T, d, f, E, K, fs = 6, 4, 5, 3, 2, 3
    cfg, inp, logits, idx, w = _rand_layer(T, d, f, E, K, seed=44, shared=fs)

    class Layer(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w1, w3, w2, ww, ws1, ws3, ws2):
            ctx.save_for_backward(x, w1, w3, w2, ww, ws1, ws3, ws2)
            return oracle.forward(x, w1, w3, w2, idx, ww, ws1, ws3, ws2)

        @staticmethod
        def backward(ctx, dy):
            x, w1, w3, w2, ww, ws1, ws3, ws2 = ctx.saved_tensors
            r = oracle.backward(x, w1, w3, w2, idx, ww, dy, ws1, ws3, ws2)
            return (r["dx"], r["dw1"], r["dw3"], r["dw2"], r["d_w"],
                    r["dws1"], r["dws3"], r["dws2"])

    ins = tuple(t.double().clone().requires_grad_() for t in
                (inp["x"], inp["w1"], inp["w3"], inp["w2"], w,
                 inp["ws1"], inp["ws3"], inp["ws2"]))
    assert torch.autograd.gradcheck(Layer.apply, ins, eps=1e-6, atol=1e-7)
