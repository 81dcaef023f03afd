"""Seeded synthetic inputs for the dropless MoE layer.

This module is the only code that both the CPU oracle's tests and the HIP path
use. It draws random tensors and builds routing workloads; it computes nothing
of the layer itself (no gating, no permutation, no expert FFN).

Workload shapes follow the models named on the pages: a tiny fp32 layer, a
Mixtral-8x7B-shaped layer, a DeepSeek-V3-shaped layer (sigmoid gating with a
route bias and one shared expert), a Qwen-MoE-like fine-grained layer (60
narrow experts, top-4, an ungated shared expert), and a skewed layer whose
router logits are synthesised so that expert loads follow a Zipf law with
some experts empty.
The pages measure no public dataset; these seeded tensors stand in for it.

Seeding: every tensor has its own generator seeded with
``seed * 1000 + tensor_index``; values are drawn in fp32 and then rounded
(round-to-nearest-even) to the layer's activation dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# tensor indices for the per-tensor seeds
_IDX = {"x": 0, "wr": 1, "bias": 2, "w1": 3, "w3": 4, "w2": 5,
        "ws1": 6, "ws3": 7, "ws2": 8, "logits": 9, "dy": 10, "zipf": 11}


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens (batch*sequence, flattened)
    d: int            # d_model
    f: int            # routed expert d_ff
    E: int            # routed experts
    K: int            # experts per token
    f_shared: int = 0  # shared expert d_ff (0 = no shared expert)
    gate: str = "softmax"   # "softmax" | "sigmoid"
    dtype: str = "bf16"     # activation / weight dtype: "f32" | "bf16"
    bias: bool = False      # route bias used for selection only
    synth_logits: bool = False  # logits synthesised (router GEMM bypassed)
    n_zero: int = 0         # synthesised: experts with zero load
    zipf_s: float = 0.0     # synthesised: Zipf exponent of the loads

    @property
    def TK(self) -> int:
        return self.T * self.K

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads. Names say what they are; sizes are the full sizes.
TINY_FP32 = MoEConfig("tiny_fp32_T256_d128_f256_E8_K2", 256, 128, 256, 8, 2,
                      dtype="f32")
MIXTRAL = MoEConfig("mixtral8x7b_T8192_d4096_f14336_E8_K2", 8192, 4096, 14336,
                    8, 2)
DEEPSEEK_V3 = MoEConfig("deepseekv3_T4096_d7168_f2048_E256_K8_sigmoid_bias_shared2048",
                        4096, 7168, 2048, 256, 8, f_shared=2048,
                        gate="sigmoid", bias=True)
SKEWED = MoEConfig("skewed_zipf1.2_T16384_d2048_f768_E128_K8", 16384, 2048,
                   768, 128, 8, synth_logits=True, n_zero=10, zipf_s=1.2)
MIXTRAL_TRAIN = MIXTRAL.replace(name="mixtral8x7b_train_fwd_bwd_T8192_d4096_f14336_E8_K2")
# A Qwen-MoE-like fine-grained layer: many narrow experts, softmax top-4,
# and one ungated shared expert twice the routed width (the pages put
# shared experts at 1-2x a routed expert's size and print no Qwen
# dimensions; d_model 2048, 60 experts of d_ff 1408 and top-4 are the
# public Qwen1.5-MoE-A2.7B layer's).
QWEN_MOE = MoEConfig("qwen_moe_like_T8192_d2048_f1408_E60_K4_shared2816",
                     8192, 2048, 1408, 60, 4, f_shared=2816)

CONFIGS = [TINY_FP32, MIXTRAL, DEEPSEEK_V3, SKEWED, MIXTRAL_TRAIN]


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _IDX[name])
    return g


def randn(shape, std: float, seed: int, name: str, dtype, device="cpu"):
    g = _gen(seed, name, device)
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def uniform(shape, lo: float, hi: float, seed: int, name: str, device="cpu"):
    g = _gen(seed, name, device)
    t = torch.rand(shape, generator=g, dtype=torch.float32, device=device)
    return t.mul_(hi - lo).add_(lo)


def zipf_loads(T: int, E: int, K: int, n_zero: int, s: float, seed: int):
    """Per-expert token-copy loads: Zipf(s) over E - n_zero experts, n_zero
    experts at zero, each load capped at T (a token picks an expert at most
    once), summing exactly to T*K. Returns an int64 numpy array [E]."""
    TK = T * K
    rng = np.random.default_rng(seed * 1000 + _IDX["zipf"])
    ids = rng.permutation(E)
    zero_ids = np.sort(ids[:n_zero])
    active = ids[n_zero:]                 # rank r+1 goes to expert active[r]
    n_act = len(active)
    if n_act * T < TK:
        raise ValueError("cannot place T*K copies with these caps")
    target = np.array([(r + 1) ** (-s) for r in range(n_act)], dtype=np.float64)
    target *= TK / target.sum()
    # water-fill the excess above the cap onto the uncapped experts
    capped = np.zeros(n_act, dtype=bool)
    for _ in range(n_act):
        over = (target > T) & ~capped
        if not over.any():
            break
        capped |= over
        excess = (target[capped] - T).sum()
        target[capped] = T
        free = ~capped
        target[free] += excess * target[free] / target[free].sum()
    base = np.floor(target).astype(np.int64)
    rem = TK - int(base.sum())
    frac = target - base
    order = sorted(range(n_act), key=lambda r: (-frac[r], r))
    for r in order:
        if rem == 0:
            break
        if base[r] < T:
            base[r] += 1
            rem -= 1
    assert rem == 0
    loads = np.zeros(E, dtype=np.int64)
    loads[active] = base
    assert loads[zero_ids].sum() == 0 and loads.sum() == TK and loads.max() <= T
    return loads


def synth_logits(T: int, E: int, K: int, n_zero: int, s: float, seed: int):
    """fp32 router logits [T, E] whose top-K per token realises zipf_loads
    exactly: chosen experts get U(2, 4), the others U(-2, 1.5)."""
    loads = zipf_loads(T, E, K, n_zero, s, seed)
    # lay the copies out expert by expert; copy i goes to token i mod T.
    # every load <= T, so no token meets the same expert twice.
    seq = np.repeat(np.arange(E), loads)
    tok = np.arange(T * K) % T
    rng = np.random.default_rng(seed * 1000 + _IDX["logits"])
    tperm = rng.permutation(T)
    chosen = np.zeros((T, E), dtype=bool)
    chosen[tperm[tok], seq] = True
    assert (chosen.sum(1) == K).all()
    hi = rng.uniform(2.0, 4.0, size=(T, E)).astype(np.float32)
    lo = rng.uniform(-2.0, 1.5, size=(T, E)).astype(np.float32)
    logits = np.where(chosen, hi, lo).astype(np.float32)
    return torch.from_numpy(logits), torch.from_numpy(loads)


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu",
                with_dy: bool = False) -> dict:
    """All layer inputs for ``cfg`` on ``device``. Weights follow the
    ``[out, in]`` linear-layer layout and are N(0, 1/fan_in)."""
    dt = cfg.torch_dtype
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    inp = {
        "x": randn((T, d), 1.0, seed, "x", dt, device),
        "wr": randn((E, d), 1.0 / math.sqrt(d), seed, "wr", dt, device),
        "w1": randn((E, f, d), 1.0 / math.sqrt(d), seed, "w1", dt, device),
        "w3": randn((E, f, d), 1.0 / math.sqrt(d), seed, "w3", dt, device),
        "w2": randn((E, d, f), 1.0 / math.sqrt(f), seed, "w2", dt, device),
        "bias": None, "logits_in": None, "loads": None,
        "ws1": None, "ws3": None, "ws2": None, "dy": None,
    }
    if cfg.bias:
        inp["bias"] = uniform((E,), -0.1, 0.1, seed, "bias", device)
    if cfg.f_shared:
        fs = cfg.f_shared
        inp["ws1"] = randn((fs, d), 1.0 / math.sqrt(d), seed, "ws1", dt, device)
        inp["ws3"] = randn((fs, d), 1.0 / math.sqrt(d), seed, "ws3", dt, device)
        inp["ws2"] = randn((d, fs), 1.0 / math.sqrt(fs), seed, "ws2", dt, device)
    if cfg.synth_logits:
        lg, loads = synth_logits(T, E, cfg.K, cfg.n_zero, cfg.zipf_s, seed)
        inp["logits_in"] = lg.to(device)
        inp["loads"] = loads
    if with_dy:
        inp["dy"] = randn((T, d), 1.0, seed, "dy", dt, device)
    return inp


def tie_logits(T: int, E: int, device="cpu") -> torch.Tensor:
    """Adversarial logits for exact-selection tests: rows of all-equal values,
    +0.0/-0.0 pairs, repeated maxima and values one ulp apart."""
    rows = []
    rng = np.random.default_rng(12345)
    for t in range(T):
        kind = t % 5
        if kind == 0:
            r = np.full(E, 0.75, dtype=np.float32)
        elif kind == 1:
            r = np.where(rng.random(E) < 0.5, np.float32(0.0),
                         np.float32(-0.0)).astype(np.float32)
        elif kind == 2:
            r = rng.choice(np.array([1.0, 2.0, 3.0], dtype=np.float32), size=E)
        elif kind == 3:
            # values a few ulps around 1.5, with repeats
            steps = rng.integers(-3, 4, size=E).astype(np.int32)
            r = (np.full(E, 1.5, dtype=np.float32).view(np.int32)
                 + steps).view(np.float32)
        else:
            r = rng.standard_normal(E).astype(np.float32)
            r[rng.integers(0, E, size=3)] = r.max()
        rows.append(r)
    return torch.from_numpy(np.stack(rows).astype(np.float32)).to(device)
