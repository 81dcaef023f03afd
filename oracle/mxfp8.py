"""fp8-aware oracle for the MXFP8 forward variant.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

[P2] (ai.warp-studio.com, section on the TE mechanisms) names a group-aware
MXFP8 grouped GEMM for the expert matmuls; [P3 §13.6] asks for per-tile
rather than per-tensor scales and fp32 accumulation. The pages give no
bit-level rule, so this follows the public OCP Microscaling (MX) v1.0 format:

  * blocks of 32 consecutive elements along each GEMM's contraction
    dimension share one E8M0 scale 2^X;
  * X = floor(log2(amax)) - 8, where 8 is the largest exponent of E4M3,
    clamped to [-127, 127]; the stored scale code is X + 127;
  * each element is v / 2^X rounded to the nearest E4M3 value (ties to an
    even mantissa) and saturated to +-448; an all-zero block gets code 0.

Both operands of all three expert GEMMs are quantised: x and W1/W3 along
d_model, h and W2 along d_ff. Products are then taken in fp64 on the
dequantised values.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

from .moe_oracle import _f64, _token_subset, swiglu

F64 = torch.float64
E4M3_MAX = 448.0
E4M3_EMAX = 8
BLOCK = 32


def e4m3_values() -> torch.Tensor:
    """Value of each of the 256 E4M3 (e4m3fn) codes from the format's
    definition: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there
    is no infinity."""
    vals = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals.append(float("nan"))
        elif e == 0:
            vals.append(s * (m / 8.0) * 2.0 ** -6)
        else:
            vals.append(s * (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return torch.tensor(vals, dtype=F64)


def e4m3_round(v: torch.Tensor) -> torch.Tensor:
    """Nearest E4M3 value to each element (fp64 in, fp64 out), ties to an
    even mantissa, saturating to +-448. In the binade [2^e, 2^(e+1)) the
    E4M3 spacing is 2^(e-3); below 2^-6 it is the subnormal step 2^-9."""
    v = _f64(v)
    a = v.abs()
    _, ex = torch.frexp(a)               # a = m * 2^ex, m in [0.5, 1)
    e = torch.clamp(ex.to(F64) - 1.0, min=-6.0)
    q = torch.pow(2.0, e - 3.0)
    r = torch.round(a / q) * q           # torch.round: half to even
    r = torch.clamp(r, max=E4M3_MAX)
    r = torch.where(a == 0, torch.zeros_like(r), r)
    return torch.copysign(r, v)


def _block_view(v: torch.Tensor, block: int):
    if v.shape[-1] % block:
        raise ValueError("last dimension must be a multiple of the block")
    return v.reshape(*v.shape[:-1], v.shape[-1] // block, block)


def mx_quantize(v: torch.Tensor, block: int = BLOCK):
    """Quantise along the last dimension. Returns (q, codes): q are the
    E4M3 element values (fp64, on the E4M3 grid) with the same shape as v;
    codes are the uint8 E8M0 scale codes, one per block."""
    vb = _block_view(_f64(v), block)
    amax = vb.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)
    X = torch.where(amax > 0, ex.to(F64) - 1.0 - E4M3_EMAX,
                    torch.full_like(amax, -127.0))
    X = torch.clamp(X, -127.0, 127.0)
    q = e4m3_round(vb / torch.pow(2.0, X).unsqueeze(-1))
    codes = (X + 127.0).to(torch.uint8)
    return q.reshape(v.shape), codes


def mx_dequantize(q: torch.Tensor, codes: torch.Tensor,
                  block: int = BLOCK) -> torch.Tensor:
    """q * 2^(code - 127) per block, fp64."""
    qb = _block_view(_f64(q), block)
    scale = torch.pow(2.0, codes.to(F64) - 127.0)
    return (qb * scale.unsqueeze(-1)).reshape(q.shape)


def mx_roundtrip(v: torch.Tensor, block: int = BLOCK) -> torch.Tensor:
    """Quantise then dequantise along the last dimension."""
    q, c = mx_quantize(v, block)
    return mx_dequantize(q, c, block)


def forward_mxfp8(x, w1, w3, w2, idx, w, ws1=None, ws3=None, ws2=None,
                  tokens: Optional[Sequence[int]] = None,
                  weight_cache: Optional[dict] = None,
                  quant: bool = True) -> torch.Tensor:
    """The [P3 §9] per-expert layer with every expert GEMM operand MX
    quantised: x and W1/W3 along d_model, h and W2 along d_ff (each along
    its GEMM's contraction, which is the last dimension of every operand
    in the [out, in] weight layout). h is quantised from its fp64 value.
    Gate weights and the combine stay in fp64. ``weight_cache`` (a dict)
    keeps dequantised weights between calls. quant=False makes every
    quantiser the identity, which must give the exact layer."""
    cache = {} if weight_cache is None else weight_cache
    Q = mx_roundtrip if quant else _f64

    def wq(name, e, t):
        key = (name, e, quant)
        if key not in cache:
            cache[key] = Q(t)
        return cache[key]

    def ffn(X, W1, W3, W2):
        a = X @ W1.T
        b = X @ W3.T
        h = Q(swiglu(a, b))
        return h @ W2.T

    sel = _token_subset(x.shape[0], tokens)
    xq = Q(_f64(x[sel]))
    idx_s = idx[sel]
    w_s = _f64(w[sel])
    out = torch.zeros(xq.shape, dtype=F64)
    for e in range(w1.shape[0]):
        mask = idx_s == e
        if not bool(mask.any()):
            continue
        rows, ks = mask.nonzero(as_tuple=True)
        Y = ffn(xq[rows], wq("w1", e, w1[e]), wq("w3", e, w3[e]),
                wq("w2", e, w2[e]))
        out.index_add_(0, rows, Y * w_s[rows, ks].unsqueeze(-1))
    if ws1 is not None:
        out += ffn(xq, wq("ws1", -1, ws1), wq("ws3", -1, ws3),
                   wq("ws2", -1, ws2))
    return out


# --------------------------------------------------------------------------
# MXFP8 backward. The pages give FP8 training as gradients times transposed
# FP8 weights with fp32 accumulation and per-tile scales [P3 §13.6.2]. Read
# with the forward's rule, both operands of each data-gradient product are
# MX quantised along that product's contraction:
#   dh = Q_d(g) . Q_d(W2)            (W2 [d, f] in blocks along d)
#   dx_perm = Q_f(da) . Q_f(W1) + Q_f(db) . Q_f(W3)   (W1 [f, d] along f)
# and fp64 products of the dequantised values. The operands that are MX
# quantised here (g = w * dy, da, db) have E8M0 codes and E4M3 elements:
# integers decided by floating point, so both sides take that decision in
# the same precision. The layer holds its intermediates in the activation
# dtype (bf16), so g, da and db are rounded to bf16 before they are
# quantised, and da, db are formed from the pre-activations a, b as the
# layer holds them, in bf16: a 2^-9 difference in a or b moves da, db
# across an E4M3 rounding boundary for about one element in 30 (one E4M3
# step, 2^-3 relative, each), about 0.03 of max|dx| in all. The weight
# gradients take the operands the forward multiplied, unquantised by the
# backward: dW2 = g^T Q_f(h), dW1 = da^T Q_d(x), dW3 = db^T Q_d(x).
# quant=False turns every quantiser and the bf16 rounding into the
# identity, which must give the exact backward.
# --------------------------------------------------------------------------

def mx_roundtrip_cols(W: torch.Tensor, block: int = BLOCK) -> torch.Tensor:
    """Quantise then dequantise a matrix in blocks of 32 along its first
    dimension (the contraction of a product that reads it transposed)."""
    return mx_roundtrip(_f64(W).T, block).T


def _bf16r(v: torch.Tensor) -> torch.Tensor:
    return v.to(torch.bfloat16).to(F64)


def _mx_bwd_ops(quant: bool):
    ident = lambda v: _f64(v)  # noqa: E731
    if not quant:
        return ident, ident, ident
    return (lambda v: mx_roundtrip(_f64(v))), mx_roundtrip_cols, _bf16r


def _mx_ffn_bwd(X, W1, W3, W2, g, Q, Qc, R):
    """One SwiGLU FFN's MXFP8 backward over rows X (already quantised) with
    output gradient g (held in bf16): (dX, dW1, dW3, dW2, Y)."""
    a = X @ Q(W1).T
    b = X @ Q(W3).T
    hq = Q(swiglu(a, b))
    Y = hq @ Q(W2).T
    dh = Q(g) @ Qc(W2)
    a, b = R(a), R(b)
    sg = torch.sigmoid(a)
    da = R(dh * b * sg * (1.0 + a * (1.0 - sg)))
    db = R(dh * a * sg)
    dX = Q(da) @ Qc(W1) + Q(db) @ Qc(W3)
    return dX, da.T @ X, db.T @ X, g.T @ hq, Y


def backward_mxfp8(x, w1, w3, w2, idx, w, dy, ws1=None, ws3=None, ws2=None,
                   quant: bool = True) -> dict:
    """Gradients of sum(dy * forward_mxfp8(...)) under the reading above,
    routing fixed and the gate weights as leaves; experts with no token
    get dW = 0. With a shared expert (ws1, ws3, ws2) it is one more FFN over
    every token, ungated (g = dy), added into dx."""
    Q, Qc, R = _mx_bwd_ops(quant)
    T, d = x.shape
    E, f, _ = w1.shape
    x64, dy64, w64 = _f64(x), _f64(dy), _f64(w)
    dx = torch.zeros(T, d, dtype=F64)
    dw1 = torch.zeros(E, f, d, dtype=F64)
    dw3 = torch.zeros_like(dw1)
    dw2 = torch.zeros(E, d, f, dtype=F64)
    d_w = torch.zeros(w.shape, dtype=F64)
    for e in range(E):
        mask = idx == e
        if not bool(mask.any()):
            continue
        rows, ks = mask.nonzero(as_tuple=True)
        g = R(dy64[rows] * w64[rows, ks].unsqueeze(-1))
        dX, dw1[e], dw3[e], dw2[e], Y = _mx_ffn_bwd(
            Q(x64[rows]), w1[e], w3[e], w2[e], g, Q, Qc, R)
        d_w[rows, ks] = (dy64[rows] * Y).sum(dim=1)
        dx.index_add_(0, rows, dX)
    res = {"dx": dx, "dw1": dw1, "dw3": dw3, "dw2": dw2, "d_w": d_w}
    if ws1 is not None:
        dX, res["dws1"], res["dws3"], res["dws2"], _ = _mx_ffn_bwd(
            Q(x64), ws1, ws3, ws2, R(dy64), Q, Qc, R)
        dx += dX
    return res


def backward_mxfp8_sampled(x, w1, w3, w2, idx, w, dy, tokens, cols) -> dict:
    """backward_mxfp8 on a sample, for full-size shapes: dx and d_w of the
    given tokens (each needs only its own K copies), and for (e, j) pairs
    row j of dW1_e and dW3_e and column j of dW2_e (hidden unit j over the
    expert's rows; Q_f(h) at j needs only j's 32-block of h). Weights are
    quantised per expert as they are needed."""
    Q, Qc, R = _mx_bwd_ops(True)
    x64, dy64, w64 = _f64(x), _f64(dy), _f64(w)
    K = idx.shape[1]
    tokens = _token_subset(x.shape[0], tokens)
    dx = torch.zeros(tokens.numel(), x.shape[1], dtype=F64)
    d_w = torch.zeros(tokens.numel(), K, dtype=F64)
    need = {}
    for i, t in enumerate(tokens.tolist()):
        for k in range(K):
            need.setdefault(int(idx[t, k]), []).append((i, t, k))
    for e, copies in sorted(need.items()):
        W1f, W3f, W2f = Q(w1[e]), Q(w3[e]), Q(w2[e])
        W1c, W3c, W2c = Qc(w1[e]), Qc(w3[e]), Qc(w2[e])
        for i, t, k in copies:
            X = Q(x64[t:t + 1])
            a, b = X @ W1f.T, X @ W3f.T
            Y = Q(swiglu(a, b)) @ W2f.T
            d_w[i, k] = (dy64[t] * Y[0]).sum()
            g = R(w64[t, k] * dy64[t:t + 1])
            dh = Q(g) @ W2c
            a, b = R(a), R(b)
            sg = torch.sigmoid(a)
            da = R(dh * b * sg * (1.0 + a * (1.0 - sg)))
            db = R(dh * a * sg)
            dx[i] += (Q(da) @ W1c + Q(db) @ W3c)[0]
        del W1f, W3f, W2f, W1c, W3c, W2c
    dw1_rows, dw3_rows, dw2_cols = [], [], []
    for e, j in cols:
        rows, ks = (idx == e).nonzero(as_tuple=True)
        X = Q(x64[rows])
        blk = slice(j - j % BLOCK, j - j % BLOCK + BLOCK)
        a = X @ Q(w1[e][blk]).T
        b = X @ Q(w3[e][blk]).T
        hq = Q(swiglu(a, b))[:, j % BLOCK]
        g = R(dy64[rows] * w64[rows, ks].unsqueeze(-1))
        dh = Q(g) @ mx_roundtrip(_f64(w2[e][:, j]))
        aj, bj = R(a[:, j % BLOCK]), R(b[:, j % BLOCK])
        sg = torch.sigmoid(aj)
        da = R(dh * bj * sg * (1.0 + aj * (1.0 - sg)))
        db = R(dh * aj * sg)
        dw1_rows.append(da @ X)
        dw3_rows.append(db @ X)
        dw2_cols.append(g.T @ hq)
    return {"dx": dx, "d_w": d_w, "dw1_rows": dw1_rows,
            "dw3_rows": dw3_rows, "dw2_cols": dw2_cols}
