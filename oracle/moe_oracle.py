"""fp64 CPU oracle of the dropless MoE layer: routing, permutation, expert
SwiGLU FFNs, combine, and the backward pass.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline). It
shares no code with the HIP library and is deliberately plain and slow: a
per-expert Python loop over torch fp64 CPU tensors.

Pages cited below:
  [P3] quant67.com, "【大模型基础设施工程】08：MoE 训练工程" (LLM infrastructure
       engineering 08: MoE training engineering); sections as numbered there.
  [P2] ai.warp-studio.com, "JAXにおけるDropless MoE訓練をNVIDIA Transformer
       Engineで劇的に加速する技術分析", section on the TE mechanisms.
  [P1] kongchang.com, "JAX中加速Dropless MoE训练：NVIDIA Transformer Engine解析",
       section "Dropless MoE：解决 token 丢弃问题".

Readings of what the pages leave open (each also listed in the design notes):
  * selection uses the fp32 logits themselves (softmax and sigmoid are
    strictly increasing, so top-K on them equals top-K on the logits);
  * ties go to the lowest expert id, also at the K-th place; the K outputs of
    a token are ordered by (key descending, id ascending); -0.0 ties +0.0;
    NaN keys count as -inf;
  * weights are always renormalised over the selected K, with no extra
    scaling; a zero sum (unreachable for finite logits) gives 1/K each;
  * the gate weight multiplies the expert output in the combine;
  * within an expert, copies keep token order (row-major nonzero).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

F64 = torch.float64


def _f64(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu", F64)


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------
def router_logits(x: torch.Tensor, wr: torch.Tensor) -> torch.Tensor:
    """logits = x Wr^T in fp64. [P3 §4.1] the gate is a bias-free linear
    layer from d_model to n_experts; [P3 §12.7] gate math is kept in fp32 or
    better."""
    return _f64(x) @ _f64(wr).T


def selection_keys(logits: torch.Tensor,
                   bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-(token, expert) selection key, as fp64 holding fp32 values.

    [P3 §6.3] and the [P3 §9] MoELayer listing add the route bias to the
    logits for selection only. The addition is done in fp32 with
    round-to-nearest-even, as on the device. -0.0 is made +0.0 and NaN is
    made -inf."""
    L = logits.detach().to("cpu", torch.float32).clone()
    if bias is not None:
        L = L + bias.detach().to("cpu", torch.float32)[None, :]
    L = torch.where(L == 0, torch.zeros_like(L), L)
    L = torch.where(torch.isnan(L), torch.full_like(L, float("-inf")), L)
    return L.to(F64)


def topk_select(keys: torch.Tensor, K: int) -> torch.Tensor:
    """The K experts of each token, ordered by (key descending, id
    ascending). [P3 §4.1] picks the top-K scores per token. A stable sort of
    the negated keys keeps ascending ids among equal keys."""
    order = np.argsort(-keys.numpy(), axis=1, kind="stable")
    return torch.from_numpy(np.ascontiguousarray(order[:, :K])).to(torch.int64)


def gate_weights(logits: torch.Tensor, idx: torch.Tensor, gate: str
                 ) -> torch.Tensor:
    """Renormalised gate weights of the selected experts, fp64.

    softmax [P3 §4.1]: softmax over all experts, keep the top-K, divide by
    their sum. The full-softmax denominator cancels, so this is a softmax
    over the selected (raw) logits.
    sigmoid [P3 §4.3, §6.3]: independent sigmoid of the raw logits of the
    selected experts, divided by their sum."""
    L = _f64(logits)
    Ls = torch.gather(L, 1, idx)
    if gate == "softmax":
        z = torch.exp(Ls - Ls.max(dim=1, keepdim=True).values)
    elif gate == "sigmoid":
        z = 1.0 / (1.0 + torch.exp(-Ls))
    else:
        raise ValueError(gate)
    s = z.sum(dim=1, keepdim=True)
    K = idx.shape[1]
    return torch.where(s > 0, z / s, torch.full_like(z, 1.0 / K))


def route(logits: torch.Tensor, K: int, gate: str,
          bias: Optional[torch.Tensor] = None):
    """(topk_idx int64 [T,K], topk_w fp64 [T,K]) from fp32 logits."""
    idx = topk_select(selection_keys(logits, bias), K)
    return idx, gate_weights(logits, idx, gate)


# --------------------------------------------------------------------------
# Permutation
# --------------------------------------------------------------------------
def permute(idx: torch.Tensor, E: int):
    """Expert-sorted order of the T*K token copies.

    Copy j = t*K + k goes to expert idx[t, k]. [P3 §9] gathers each expert's
    tokens with a row-major nonzero of (topk_idx == e), i.e. in increasing
    j; [P3 §9] also counts the load per expert. Returns counts [E],
    offsets [E+1] (exclusive prefix sum), sorted_src [T*K] (the j at each
    sorted position) and dest [T*K] (the sorted position of each j)."""
    flat = idx.reshape(-1).to(torch.int64)
    TK = flat.numel()
    counts = torch.zeros(E, dtype=torch.int64)
    parts = []
    for e in range(E):
        js = (flat == e).nonzero().flatten()
        counts[e] = js.numel()
        parts.append(js)
    offsets = torch.zeros(E + 1, dtype=torch.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_src = torch.cat(parts) if parts else torch.zeros(0, dtype=torch.int64)
    dest = torch.empty(TK, dtype=torch.int64)
    dest[sorted_src] = torch.arange(TK)
    return counts, offsets, sorted_src, dest


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------
def _sigmoid(a: torch.Tensor) -> torch.Tensor:
    return 1.0 / (1.0 + torch.exp(-a))


def swiglu(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """silu(a) * b with silu(a) = a * sigmoid(a). [P3 §9] Expert."""
    return a * _sigmoid(a) * b


def expert_ffn(X: torch.Tensor, W1, W3, W2):
    """One SwiGLU expert, [P3 §9] Expert: w2(silu(w1 x) * w3 x), weights in
    the [out, in] linear-layer layout. Returns (a, b, h, Y), all fp64."""
    X = _f64(X)
    a = X @ _f64(W1).T
    b = X @ _f64(W3).T
    h = swiglu(a, b)
    Y = h @ _f64(W2).T
    return a, b, h, Y


def _token_subset(T: int, tokens) -> torch.Tensor:
    if tokens is None:
        return torch.arange(T)
    return torch.as_tensor(tokens, dtype=torch.int64)


def forward(x, w1, w3, w2, idx, w, ws1=None, ws3=None, ws2=None,
            tokens: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Layer output [len(tokens), d] in fp64.

    [P3 §9] MoELayer.forward: for each expert with any token, gather its
    tokens, run the expert, scale by the gate weight and index_add into the
    output; experts with no token are skipped. [P3 §5] then adds the
    shared expert, ungated, for every token. Each output row depends only
    on its own token, so ``tokens`` restricts the work to a subset."""
    sel = _token_subset(x.shape[0], tokens)
    xs = _f64(x[sel])
    idx_s = idx[sel]
    w_s = _f64(w[sel])
    out = torch.zeros(xs.shape[0], xs.shape[1], dtype=F64)
    for e in range(w1.shape[0]):
        mask = idx_s == e
        if not bool(mask.any()):
            continue
        rows, ks = mask.nonzero(as_tuple=True)
        Y = expert_ffn(xs[rows], w1[e], w3[e], w2[e])[3]
        out.index_add_(0, rows, Y * w_s[rows, ks].unsqueeze(-1))
    if ws1 is not None:
        out += expert_ffn(xs, ws1, ws3, ws2)[3]
    return out


def forward_gather(x, w1, w3, w2, idx, w, ws1=None, ws3=None, ws2=None):
    """Second formulation of the same layer, from the [P3 §12.5] EP listing
    with one rank (every all-to-all is the identity): sort the flattened
    copies by expert, gather the token rows, run each expert on its
    contiguous slice, weight, undo the sort, and sum the K copies."""
    T, d = x.shape
    K = idx.shape[1]
    flat_idx = idx.reshape(-1)
    sort_perm = torch.sort(flat_idx, stable=True).indices
    sorted_tok = _f64(x).repeat_interleave(K, dim=0)[sort_perm]
    sorted_expert = flat_idx[sort_perm]
    sorted_weight = _f64(w).reshape(-1)[sort_perm]
    out_local = torch.zeros_like(sorted_tok)
    for e in range(w1.shape[0]):
        m = sorted_expert == e
        if bool(m.any()):
            out_local[m] = expert_ffn(sorted_tok[m], w1[e], w3[e], w2[e])[3]
    back = out_local * sorted_weight.unsqueeze(-1)
    unsort = torch.empty_like(sort_perm)
    unsort[sort_perm] = torch.arange(sort_perm.numel())
    out = back[unsort].view(T, K, d).sum(dim=1)
    if ws1 is not None:
        out = out + expert_ffn(_f64(x), ws1, ws3, ws2)[3]
    return out


def dense_masked_forward(x, w1, w3, w2, idx, w, ws1=None, ws3=None, ws2=None):
    """Brute force for tiny inputs: every expert on every token, summed with
    a dense [T, E] gate matrix that is zero off the routed experts."""
    T = x.shape[0]
    E = w1.shape[0]
    G = torch.zeros(T, E, dtype=F64)
    for t in range(T):
        for k in range(idx.shape[1]):
            G[t, int(idx[t, k])] += float(w[t, k])
    out = torch.zeros(T, x.shape[1], dtype=F64)
    for e in range(E):
        out += G[:, e:e + 1] * expert_ffn(x, w1[e], w3[e], w2[e])[3]
    if ws1 is not None:
        out += expert_ffn(x, ws1, ws3, ws2)[3]
    return out


# --------------------------------------------------------------------------
# Per-stage definitions (for checking each kernel on its own inputs)
# --------------------------------------------------------------------------
def _rows_by_expert(offsets: torch.Tensor, rows):
    """Map sorted positions to their experts using offsets."""
    off = offsets.to(torch.int64)
    rows = torch.as_tensor(rows, dtype=torch.int64)
    e_of = torch.searchsorted(off[1:], rows, right=True)
    return rows, e_of


def stage_gemm1(x_perm, offsets, w1, w3, rows=None):
    """Sorted rows p of expert e: a = x_perm[p] W1_e^T, b = x_perm[p] W3_e^T,
    h = silu(a) * b ([P3 §9] Expert, first half). Returns (a, b, h) fp64
    for the requested rows (all by default)."""
    TK = x_perm.shape[0]
    rows, e_of = _rows_by_expert(offsets, range(TK) if rows is None else rows)
    f = w1.shape[1]
    a = torch.zeros(rows.numel(), f, dtype=F64)
    b = torch.zeros_like(a)
    for e in torch.unique(e_of).tolist():
        m = e_of == e
        X = _f64(x_perm[rows[m]])
        a[m] = X @ _f64(w1[e]).T
        b[m] = X @ _f64(w3[e]).T
    return a, b, swiglu(a, b)


def stage_gemm2(h_perm, offsets, w2, rows=None):
    """y_perm[p] = h_perm[p] W2_e^T for sorted rows p of expert e."""
    TK = h_perm.shape[0]
    rows, e_of = _rows_by_expert(offsets, range(TK) if rows is None else rows)
    y = torch.zeros(rows.numel(), w2.shape[1], dtype=F64)
    for e in torch.unique(e_of).tolist():
        m = e_of == e
        y[m] = _f64(h_perm[rows[m]]) @ _f64(w2[e]).T
    return y


def stage_combine(y_perm, dest, w, y_shared=None, tokens=None):
    """out[t] = sum_k w[t,k] * y_perm[dest[t*K+k]] (+ y_shared[t]): [P3 §12.5]
    step 6 (weight, undo the sort, sum over K) plus [P3 §5]."""
    T, K = w.shape
    sel = _token_subset(T, tokens)
    dest = dest.to(torch.int64).view(T, K)
    out = torch.zeros(sel.numel(), y_perm.shape[1], dtype=F64)
    for k in range(K):
        out += _f64(w[sel, k]).unsqueeze(-1) * _f64(y_perm[dest[sel, k]])
    if y_shared is not None:
        out += _f64(y_shared[sel])
    return out


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------
def _swiglu_bwd(a, b, dh):
    """d/da and d/db of silu(a) * b: silu'(a) = s (1 + a (1 - s))."""
    s = _sigmoid(a)
    da = dh * b * s * (1.0 + a * (1.0 - s))
    db = dh * a * s
    return da, db


def backward(x, w1, w3, w2, idx, w, dy, ws1=None, ws3=None, ws2=None):
    """Gradients of sum(dy * forward(...)) with routing fixed and the gate
    weights w as leaves. [P3 §11.3]: only experts that received tokens get
    gradient; an expert with none gets dW = 0.

    Per expert e with copies (t, k):
      Y = expert output (unweighted);  d_w[t,k] = <dy[t], Y>
      g = w[t,k] dy[t];  dW2_e = g^T h;  dh = g W2_e
      da, db from the SwiGLU derivative;  dW1_e = da^T X;  dW3_e = db^T X
      dX[t] += da W1_e + db W3_e
    plus the same for the ungated shared expert over all tokens."""
    T, d = x.shape
    E, f, _ = w1.shape
    x64 = _f64(x)
    dy64 = _f64(dy)
    w64 = _f64(w)
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
        X = x64[rows]
        W1, W3, W2 = _f64(w1[e]), _f64(w3[e]), _f64(w2[e])
        a, b, h, Y = expert_ffn(X, W1, W3, W2)
        d_w[rows, ks] = (dy64[rows] * Y).sum(dim=1)
        g = dy64[rows] * w64[rows, ks].unsqueeze(-1)
        dw2[e] = g.T @ h
        da, db = _swiglu_bwd(a, b, g @ W2)
        dw1[e] = da.T @ X
        dw3[e] = db.T @ X
        dx.index_add_(0, rows, da @ W1 + db @ W3)
    res = {"dx": dx, "dw1": dw1, "dw3": dw3, "dw2": dw2, "d_w": d_w}
    if ws1 is not None:
        S1, S3, S2 = _f64(ws1), _f64(ws3), _f64(ws2)
        a, b, h, _ = expert_ffn(x64, S1, S3, S2)
        da, db = _swiglu_bwd(a, b, dy64 @ S2)
        res["dws2"] = dy64.T @ h
        res["dws1"] = da.T @ x64
        res["dws3"] = db.T @ x64
        dx += da @ S1 + db @ S3
    return res


def backward_sampled(x, w1, w3, w2, idx, w, dy, tokens, cols,
                     ws1=None, ws3=None, ws2=None):
    """The closed form of ``backward`` evaluated on a sample, for shapes
    where the full gradients are too costly on a CPU.

    tokens: token ids -> dx[tokens] and d_w[tokens] (each row needs only
            its own token's K copies).
    cols:   (e, j) pairs with 0 <= j < d_ff -> dW1_e[j, :], dW3_e[j, :]
            and dW2_e[:, j]. Column j of the expert's hidden layer needs
            a[:, j], b[:, j] and dh[:, j] over the expert's tokens only."""
    x64 = _f64(x)
    dy64 = _f64(dy)
    w64 = _f64(w)
    tokens = _token_subset(x.shape[0], tokens)
    K = idx.shape[1]
    dx = torch.zeros(tokens.numel(), x.shape[1], dtype=F64)
    d_w = torch.zeros(tokens.numel(), K, dtype=F64)
    for i, t in enumerate(tokens.tolist()):
        xt = x64[t:t + 1]
        for k in range(K):
            e = int(idx[t, k])
            W1, W3, W2 = _f64(w1[e]), _f64(w3[e]), _f64(w2[e])
            a, b, h, Y = expert_ffn(xt, W1, W3, W2)
            d_w[i, k] = (dy64[t] * Y[0]).sum()
            g = w64[t, k] * dy64[t:t + 1]
            da, db = _swiglu_bwd(a, b, g @ W2)
            dx[i] += (da @ W1 + db @ W3)[0]
        if ws1 is not None:
            S1, S3, S2 = _f64(ws1), _f64(ws3), _f64(ws2)
            a, b, h, _ = expert_ffn(xt, S1, S3, S2)
            da, db = _swiglu_bwd(a, b, dy64[t:t + 1] @ S2)
            dx[i] += (da @ S1 + db @ S3)[0]
    dw1_rows, dw3_rows, dw2_cols = [], [], []
    for e, j in cols:
        mask = idx == e
        rows, ks = mask.nonzero(as_tuple=True)
        if rows.numel() == 0:
            dw1_rows.append(torch.zeros(x.shape[1], dtype=F64))
            dw3_rows.append(torch.zeros(x.shape[1], dtype=F64))
            dw2_cols.append(torch.zeros(x.shape[1], dtype=F64))
            continue
        X = x64[rows]
        a = X @ _f64(w1[e, j])
        b = X @ _f64(w3[e, j])
        h = swiglu(a, b)
        g = dy64[rows] * w64[rows, ks].unsqueeze(-1)
        dh = g @ _f64(w2[e, :, j])
        da, db = _swiglu_bwd(a, b, dh)
        dw1_rows.append(da @ X)
        dw3_rows.append(db @ X)
        dw2_cols.append(g.T @ h)
    return {"dx": dx, "d_w": d_w, "dw1_rows": dw1_rows,
            "dw3_rows": dw3_rows, "dw2_cols": dw2_cols}


# --------------------------------------------------------------------------
# Router backward: the gate-weight gradient through the gate to the logits,
# the router weights and the tokens. The selection is piecewise constant,
# so only the K selected logits of a token receive gradient.
# --------------------------------------------------------------------------

def gate_logit_grad(logits: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                    d_w: torch.Tensor, gate: str) -> torch.Tensor:
    """d loss / d logits [T, E] (fp64) from d loss / d topk_w [T, K].

    softmax [P3 §4.1]: w = softmax over the selected logits, so
    dL_k = w_k (d_w_k - sum_j w_j d_w_j) on the selected experts.
    sigmoid [P3 §4.3]: w_k = s_k / S with s = sigmoid(L), S = sum of the
    selected s, so dL_m = s_m (1 - s_m) / S * (d_w_m - sum_k w_k d_w_k).
    A token whose weights fell back to 1/K (all selected sigmoids zero) has
    a constant gate and gets zero gradient."""
    L = _f64(logits)
    idx = idx.to(torch.int64)
    w = _f64(w)
    d_w = _f64(d_w)
    Ls = torch.gather(L, 1, idx)
    inner = (w * d_w).sum(dim=1, keepdim=True)
    if gate == "softmax":
        g = w * (d_w - inner)
    elif gate == "sigmoid":
        s = _sigmoid(Ls)
        S = s.sum(dim=1, keepdim=True)
        g = torch.where(S > 0, s * (1.0 - s) / torch.where(S > 0, S, 1.0)
                        * (d_w - inner), torch.zeros_like(s))
    else:
        raise ValueError(gate)
    out = torch.zeros_like(L)
    out.scatter_(1, idx, g)
    return out


def router_backward(x, wr, logits, idx, w, d_w, gate: str,
                    aux_coef: float = 0.0):
    """Gradients of the router: d_logits [T, E], d_wr = d_logits^T x
    [E, d] and the router's share of dx, d_logits wr [T, d] (fp64).
    With aux_coef != 0 the loss also holds aux_coef times the balance loss
    of load_balance_stats, whose logit gradient is added first."""
    dl = gate_logit_grad(logits, idx, w, d_w, gate)
    if aux_coef != 0.0:
        dl = dl + aux_coef * aux_loss_logit_grad(logits, idx, logits.shape[1],
                                                 gate)
    return {"d_logits": dl, "d_wr": dl.T @ _f64(x), "dx": dl @ _f64(wr)}


# --------------------------------------------------------------------------
# Load-balance statistics [P3 §6.2, §9]: the GShard-style auxiliary loss
# N * sum_i f_i P_i, with f_i the share of tokens whose top-K mask holds
# expert i and P_i the mean gate probability of expert i over the tokens.
# --------------------------------------------------------------------------

def gate_probs(logits: torch.Tensor, gate: str) -> torch.Tensor:
    """Per-token gate probabilities over all E experts [T, E] (fp64):
    softmax of the logits (softmax gate), or the sigmoids normalised to sum
    to one over all experts (sigmoid gate; raw logits, no route bias)."""
    L = _f64(logits)
    if gate == "softmax":
        return torch.softmax(L, dim=1)
    if gate == "sigmoid":
        s = _sigmoid(L)
        return s / s.sum(dim=1, keepdim=True)
    raise ValueError(gate)


def load_balance_stats(logits: torch.Tensor, idx: torch.Tensor, E: int,
                       gate: str) -> dict:
    """f [E] = mean over tokens of the top-K mask (sums to K), p_mean [E] =
    mean over tokens of the gate probabilities (sums to 1), aux = E *
    sum_i f_i p_mean_i. The load statistic of the layer [P3 §9] is f / K."""
    T = logits.shape[0]
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask.scatter_(1, idx.to(torch.int64), 1.0)
    f = mask.mean(dim=0)
    P = gate_probs(logits, gate).mean(dim=0)
    return {"f": f, "p_mean": P, "aux": E * (f * P).sum()}


def aux_loss_logit_grad(logits: torch.Tensor, idx: torch.Tensor, E: int,
                        gate: str) -> torch.Tensor:
    """d aux / d logits [T, E] (fp64), with the mask share f held constant
    (it is piecewise constant in the logits).

    aux = (E / T) sum_t sum_i f_i P_ti, so d aux / d L_tj =
    (E / T) sum_i f_i dP_ti / dL_tj. Softmax: dP_ti / dL_tj =
    P_ti (delta_ij - P_tj), giving (E / T) P_tj (f_j - sum_i f_i P_ti).
    Normalised sigmoid, P_ti = s_ti / S_t: dP_ti / dL_tj =
    s_tj (1 - s_tj) / S_t (delta_ij - P_ti), giving
    (E / T) s_tj (1 - s_tj) / S_t (f_j - sum_i f_i P_ti)."""
    L = _f64(logits)
    T = L.shape[0]
    f = load_balance_stats(L, idx, E, gate)["f"]
    P = gate_probs(L, gate)
    inner = (P * f).sum(dim=1, keepdim=True)
    if gate == "softmax":
        q = P
    else:
        s = _sigmoid(L)
        q = s * (1.0 - s) / s.sum(dim=1, keepdim=True)
    return (E / T) * q * (f - inner)


# --------------------------------------------------------------------------
# Bias-balance update and load monitor [P3 §6.3, §9, §13.9].
# Computed in fp32, in the order the definitions give, because the sign of
# (load - target) and the cold-expert count are decisions that must come
# out the same as on the device.
# --------------------------------------------------------------------------

def update_route_bias(bias, counts, gamma: float, target: float = 0.0,
                      rule: int = 0):
    """One step of the auxiliary-loss-free balancing. load = counts /
    sum(counts) (the layer's load statistic); target <= 0 means 1/E.
    rule 0 [P3 §6.3 text]: an overloaded expert's bias drops by gamma, an
    underloaded one's rises by gamma, one on target keeps it.
    rule 1 [P3 §9 update_balance_bias]: the step is additionally scaled by
    the load, clamped below at 1e-6.
    Returns (new bias, load), fp32 numpy arrays."""
    c = np.asarray(counts, dtype=np.int64)
    E = c.shape[0]
    load = c.astype(np.float32) / np.float32(c.sum())
    tgt = np.float32(target) if target > 0 else np.float32(1.0) / np.float32(E)
    sgn = np.sign(load - tgt).astype(np.float32)
    step = np.float32(gamma) * sgn
    if rule == 1:
        step = step * np.maximum(load, np.float32(1e-6))
    return (np.asarray(bias, dtype=np.float32) - step).astype(np.float32), load


def balance_monitor(load_hist):
    """Monitor figures from a window of load vectors [W, E] (oldest
    first): the mean load r over the window (fp32, summed in row order),
    its minimum, the entropy -sum r log(r + 1e-9) and the number of cold
    experts (r < 0.3 / E). Returns (min, entropy, cold) as floats."""
    h = np.asarray(load_hist, dtype=np.float32)
    W, E = h.shape
    s = np.zeros(E, dtype=np.float32)
    for w in range(W):
        s = (s + h[w]).astype(np.float32)
    r = (s / np.float32(W)).astype(np.float32)
    r64 = r.astype(np.float64)
    entropy = float(-(r64 * np.log(r64 + 1e-9)).sum())
    cold = int((r < np.float32(0.3) / np.float32(E)).sum())
    return float(r.min()), entropy, cold
