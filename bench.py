"""Benchmark of the dropless MoE layer forward on one MI355X.

A step is one whole forward of the layer (router GEMM, top-K gate,
histogram/scan/permute, grouped SwiGLU GEMM 1, grouped GEMM 2, combine) on
one batch of seeded synthetic input already resident in HBM. Three input
batches rotate so no step reuses the previous step's activations from the
last-level cache. The default workload is the Mixtral-8x7B-shaped layer
(T=8192, d_model=4096, d_ff=14336, E=8, top-2 softmax, bf16).

Prints ONE JSON line. Per-stage times come from HIP events the library
records on the launch stream between its kernels; the roofline object
reports the dominant kernel (grouped GEMM 1 + SwiGLU) against the bf16
MFMA peak; the CPU baseline times the fp64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer fwd TFLOP/s (routed FLOPs) + % bf16 MFMA peak; "
          "permute GB/s")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector (the fp32 path runs on VALU)

# Bytes per launch of grouped GEMM 1 + SwiGLU on the Mixtral-shaped layer,
# from rocprofv3 FETCH_SIZE and WRITE_SIZE passes, scaled by what the same
# counters read for a 1 GiB device copy (FETCH x2, WRITE x1). They describe
# the kernel built from sources with this digest and nothing else.
GEMM1_TRAFFIC = {
    "workload": "mixtral8x7b_T8192_d4096_f14336_E8_K2",
    "src_digest": "03584a3f922ad71f",
    "fetch_bytes": 13_179_877_376,
    "write_bytes": 469_981_184,
}
GEMM_SOURCES = ("gemm_mfma.hip", "common.h", "gemm.h", "tile_map.h")


def gemm_src_digest():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "ragged_grouped_gemm_router_amd", "csrc",
                               f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm1_traffic(cfg, mxfp8):
    """Counter-derived bytes per launch, or None when they do not describe
    the kernel this run timed (another workload, MXFP8, changed sources)."""
    t = GEMM1_TRAFFIC
    if mxfp8 or cfg.name != t["workload"] or gemm_src_digest() != t["src_digest"]:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (recorded by the library on its stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")  # the copy torch already loaded
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [
            ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def record(self, i, stream):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        assert self.hip.hipEventRecord(self.ev[i], stream.cuda_stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a],
                                          self.ev[b])
        assert st == 0, st
        return out.value


def workload(name):
    import moe_inputs as mi
    table = {"mixtral": mi.MIXTRAL, "deepseek": mi.DEEPSEEK_V3,
             "skewed": mi.SKEWED, "qwen": mi.QWEN_MOE, "tiny": mi.TINY_FP32}
    return table[name]


def cpu_baseline(cfg, ginp, logits_gpu, n_tokens):
    """Time the fp64 oracle forward (weight upcast included) on the first
    n_tokens tokens, on the host cores. D2H copies happen before timing."""
    import torch
    import oracle
    affinity = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    # threads: every CPU this process may run on, capped by OMP_NUM_THREADS
    # when the host sets it (the CPU share of one GPU on a shared host)
    threads = min(affinity, int(omp)) if omp else affinity
    torch.set_num_threads(threads)
    toks = list(range(n_tokens))
    c = {k: (v.cpu() if isinstance(v, torch.Tensor) else v)
         for k, v in ginp.items() if k in ("x", "w1", "w3", "w2", "bias",
                                           "ws1", "ws3", "ws2")}
    logits = (ginp["logits_in"] if ginp.get("logits_in") is not None
              else logits_gpu)[:n_tokens].cpu()
    t0 = time.perf_counter()
    idx, w = oracle.route(logits, cfg.K, cfg.gate, c.get("bias"))
    oracle.forward(c["x"][:n_tokens], c["w1"], c["w3"], c["w2"], idx, w,
                   c.get("ws1"), c.get("ws3"), c.get("ws2"), tokens=toks)
    dt = time.perf_counter() - t0
    from ragged_grouped_gemm_router_amd import accounting as acc
    flops = acc.routed_fwd_flops(cfg.d, cfg.f, n_tokens * cfg.K)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "threads": torch.get_num_threads(), "host_cores": os.cpu_count(),
            "affinity_cpus": affinity,
            "threads_cap": ("OMP_NUM_THREADS=" + omp) if omp else None,
            "kind": "oracle",
            "sample": (f"first {n_tokens} tokens ({n_tokens * cfg.K} routed "
                       f"copies) of {cfg.name}; fp64 torch CPU per-expert "
                       f"loop incl. weight upcast; {dt:.1f} s")}


def graph_replay(step, stream, n_rep):
    """The same step captured once per input batch in a HIP graph, then
    replayed n_rep times in batch rotation; each replay timed with HIP
    events on the launch stream. Returns the replay times' median and
    p10 / p90 in ms."""
    import numpy as np
    import torch
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for j in range(3):
            step(0, False, j=j)  # warm the side stream (no events)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    for j in range(3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(0, False, j=j)
        graphs.append(g)
    torch.cuda.synchronize()
    for j in range(3):  # untimed first replays
        graphs[j].replay()
    torch.cuda.synchronize()
    gev = HipEvents(2 * n_rep)
    for r in range(n_rep):
        gev.record(2 * r, stream)
        graphs[r % 3].replay()
        gev.record(2 * r + 1, stream)
    torch.cuda.synchronize()
    t = np.array([gev.ms(2 * r, 2 * r + 1) for r in range(n_rep)])
    q = np.percentile(t, [10, 50, 90])
    return {"median_ms": round(float(q[1]), 4), "p10_ms": round(float(q[0]), 4),
            "p90_ms": round(float(q[2]), 4), "replays": n_rep,
            "what": "the whole step captured once per input batch in a HIP "
                    "graph and replayed in rotation"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral",
                    choices=["mixtral", "deepseek", "skewed", "qwen", "tiny"])
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens of the workload the fp64 oracle runs for the "
                         "CPU baseline, at most all of them (the whole "
                         "Mixtral-shaped workload: about 7 s on 16 host cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-replays", type=int, default=20,
                    help="after the timed steps, replay the step captured in "
                         "a HIP graph this many times (0: skip)")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step: forward (activations saved) "
                         "plus backward; FLOPs counted as 3x the forward")
    ap.add_argument("--gather", action="store_true",
                    help="forward only: leave x_perm out, GEMM 1 gathers its "
                         "rows from x through sorted_src")
    ap.add_argument("--aux-coef", type=float, default=0.01,
                    help="coefficient of the balance loss in the training "
                         "step's router backward")
    ap.add_argument("--mxfp8", action="store_true",
                    help="expert GEMMs on MXFP8 operands (weights quantised "
                         "once, before timing)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first "
                         "(a known-size kernel to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this implementation runs on one GPU only; --gpus {args.gpus} "
              "is not supported (the layer does not shard across GPUs here)",
              file=sys.stderr)
        sys.exit(2)
    if args.gather and args.backward:
        ap.error("--gather is forward only: the backward reads x_perm")

    import torch
    import moe_inputs as mi
    from ragged_grouped_gemm_router_amd import accounting as acc
    from ragged_grouped_gemm_router_amd import binding as B
    from ragged_grouped_gemm_router_amd import layer as L

    cfg = workload(args.workload)
    dev = "cuda"
    log(f"bench: workload {cfg.name}")
    base = mi.make_inputs(cfg, 0, device=dev)
    batches = [base]
    for s in (1, 2):
        b = dict(base)
        b["x"] = mi.randn((cfg.T, cfg.d), 1.0, s, "x", cfg.torch_dtype, dev)
        if cfg.synth_logits:
            lg, _ = mi.synth_logits(cfg.T, cfg.E, cfg.K, cfg.n_zero,
                                    cfg.zipf_s, s)
            b["logits_in"] = lg.to(dev)
        batches.append(b)
    desc = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, cfg.f_shared,
                       cfg.gate, cfg.dtype, mxfp8=args.mxfp8,
                       save_acts=args.backward)
    gbufs = None
    if args.backward:
        for s, b in enumerate(batches):
            b["dy"] = mi.randn((cfg.T, cfg.d), 1.0, s, "dy", cfg.torch_dtype,
                               dev)
        gbufs = [L.alloc_backward(desc, dev) for _ in batches]
        rbufs = [L.alloc_router_backward(desc, dev) for _ in batches]
        bev = HipEvents(B.MOE_BWD_NEVENTS * max(args.steps, 1))
        rev = HipEvents(3 * max(args.steps, 1))
    if args.mxfp8:
        mx = L.quantize_expert_weights(base)
        mxb = L.quantize_expert_weights_bwd(base) if args.backward else None
        for b in batches:
            b["mx"] = mx
            b["mx_bwd"] = mxb
        torch.cuda.synchronize()
    bufs = [L.alloc_forward(desc, dev, gather=args.gather) for _ in batches]
    n_steps = args.warmup + args.steps
    ev = HipEvents(B.MOE_FWD_NEVENTS * max(args.steps, 1))
    stream = torch.cuda.current_stream()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    sev = HipEvents(2 * max(args.steps, 1))  # around each whole step

    def step(i, timed, j=None, stage_events=True):
        j = i % 3 if j is None else j
        timed_stages = timed and stage_events
        if timed:
            sev.record(2 * i, stream)
        e = (ev.ev[i * B.MOE_FWD_NEVENTS:(i + 1) * B.MOE_FWD_NEVENTS]
             if timed_stages else None)
        L.forward(desc, batches[j], bufs[j], events=e)
        if args.backward:
            be = (bev.ev[i * B.MOE_BWD_NEVENTS:(i + 1) * B.MOE_BWD_NEVENTS]
                  if timed_stages else None)
            L.backward(desc, batches[j], bufs[j], batches[j]["dy"], gbufs[j],
                       events=be)
            if not cfg.synth_logits:
                # balance statistics of the routing, then the router
                # backward: the gate (and the balance loss) to Wr and dx
                if timed_stages:
                    rev.record(3 * i, stream)
                L.load_balance_stats(desc, bufs[j], rbufs[j])
                if timed_stages:
                    rev.record(3 * i + 1, stream)
                L.router_backward(desc, batches[j], bufs[j], gbufs[j],
                                  rbufs[j], aux_coef=args.aux_coef)
                if timed_stages:
                    rev.record(3 * i + 2, stream)
        if timed:
            sev.record(2 * i + 1, stream)

    log("bench: warmup")
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    log("bench: timed steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / max(args.steps, 1) * 1e3
    log(f"bench: {ms_step:.3f} ms/step")
    step_ms = [sev.ms(2 * i, 2 * i + 1) for i in range(args.steps)]
    graph = graph_replay(step, stream, args.graph_replays) \
        if args.graph_replays > 0 else None

    n = B.MOE_FWD_NEVENTS
    stage = {"route": 0.0, "permute": 0.0, "gemm1_swiglu": 0.0,
             "gemm2_shared": 0.0, "combine": 0.0}
    for i in range(args.steps):
        o = i * n
        stage["route"] += ev.ms(o + 0, o + 1)
        stage["permute"] += ev.ms(o + 1, o + 2)
        stage["gemm1_swiglu"] += ev.ms(o + 2, o + 3)
        stage["gemm2_shared"] += ev.ms(o + 3, o + 4)
        stage["combine"] += ev.ms(o + 4, o + 5)
    stage = {k: v / args.steps for k, v in stage.items()}
    bstage = None
    if args.backward:
        names = ["combine_bwd", "recompute", "dgrad2_swiglu_bwd", "dgrad1",
                 "gather_sum_dx", "wgrad_w2", "wgrad_w1_w3"]
        bstage = dict.fromkeys(names, 0.0)
        for i in range(args.steps):
            o = i * B.MOE_BWD_NEVENTS
            for q, nm in enumerate(names):
                bstage[nm] += bev.ms(o + q, o + q + 1) / args.steps
        if not cfg.synth_logits:
            bstage["balance_stats"] = sum(
                rev.ms(3 * i, 3 * i + 1) for i in range(args.steps)) / args.steps
            bstage["router_backward"] = sum(
                rev.ms(3 * i + 1, 3 * i + 2) for i in range(args.steps)) / args.steps

    TK = cfg.TK
    b = 4 if cfg.dtype == "f32" else 2
    routed = acc.routed_fwd_flops(cfg.d, cfg.f, TK)
    g1 = acc.gemm1_flops(cfg.d, cfg.f, TK)
    step_flops = acc.train_flops(routed) if args.backward else routed
    value = step_flops / (ms_step * 1e-3) / 1e12
    gemm_s = (stage["gemm1_swiglu"] + stage["gemm2_shared"]) * 1e-3
    if args.gather:  # indices only (and, under MXFP8, x quantised once)
        perm_bytes = acc.permute_index_bytes(cfg.T, cfg.K) + (
            acc.quantize_bytes(cfg.T * cfg.d) if args.mxfp8 else 0)
    else:
        perm_bytes = acc.permute_bytes(cfg.T, cfg.K, cfg.d, b)
    comb_bytes = acc.combine_bytes(cfg.T, cfg.K, cfg.d, b, cfg.f_shared > 0)
    k5_s = stage["gemm1_swiglu"] * 1e-3
    k5_tflops = g1 / k5_s / 1e12
    peak = (PEAK_FP8_TFLOPS if args.mxfp8 else
            PEAK_FP32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS)
    g1_bytes = acc.gemm1_bytes(cfg.E, cfg.d, cfg.f, TK,
                               1 + 1 / 32 if args.mxfp8 else b)
    # GEMM 1's own arithmetic intensity decides its bound: the weight
    # stream dominates when few rows share each expert (DeepSeek-V3 shape).
    if g1 / g1_bytes < peak * 1e12 / (PEAK_HBM_GBPS * 1e9):
        k5_roof = {"bound": "hbm",
                   "achieved": round(g1_bytes / k5_s / 1e9, 1),
                   "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                   "frac": round(g1_bytes / k5_s / 1e9 / PEAK_HBM_GBPS, 4)}
    else:
        k5_roof = {"bound": "mfma", "achieved": round(k5_tflops, 2),
                   "peak": peak, "unit": "TFLOP/s",
                   "frac": round(k5_tflops / peak, 4)}
    metric = METRIC
    if args.backward:
        metric = ("MoE layer training step (fwd+bwd) TFLOP/s, FLOPs = 3x "
                  "routed forward")
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp8" if args.mxfp8 else
                  "f32" if cfg.dtype == "f32" else "bf16"),
        "data": "synthetic: seeded N(0,1) tokens, N(0,1/fan_in) random-init "
                "weights" + (", Zipf-synthesised router logits"
                             if cfg.synth_logits else ""),
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d,
                   "d_ff": cfg.f, "E": cfg.E, "K": cfg.K,
                   "d_ff_shared": cfg.f_shared, "gate": cfg.gate,
                   "x_perm": "gathered in GEMM 1" if args.gather else
                             "materialised",
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "grouped_gemm_tflops": round(routed / gemm_s / 1e12, 2),
        "permute_GBps": round(perm_bytes / (stage["permute"] * 1e-3) / 1e9, 1),
        "combine_GBps": round(comb_bytes / (stage["combine"] * 1e-3) / 1e9, 1),
        "stages_ms": {k: round(v, 4) for k, v in stage.items()},
        "stages_ms_backward": ({k: round(v, 4) for k, v in bstage.items()}
                               if bstage else None),
        "roofline": {
            "kernel": "grouped GEMM 1 + SwiGLU (dual B: W1 and W3)",
            **k5_roof,
            "algorithmic_bytes": int(g1_bytes),
            "algorithmic_flops": g1,
            "traffic": (None if args.gather
                        else gemm1_traffic(cfg, args.mxfp8)),
        },
    }
    if step_ms:
        import numpy as np
        q = np.percentile(np.array(step_ms), [10, 50, 90])
        line["step_ms_events"] = {"p10": round(float(q[0]), 4),
                                  "median": round(float(q[1]), 4),
                                  "p90": round(float(q[2]), 4),
                                  "n": len(step_ms)}
    line["graph_replay"] = graph
    if args.mxfp8:
        # the MXFP8 layer against the bf16 one on the same batch (both from
        # this library, outside the timed region; the bf16 layer is held
        # to the exact fp64 oracle within 1e-2 by the parity tests)
        dbf = B.make_desc(cfg.T, cfg.d, cfg.f, cfg.E, cfg.K, cfg.f_shared,
                          cfg.gate, cfg.dtype)
        bb = {k: v for k, v in batches[0].items() if k not in ("mx", "mx_bwd")}
        fb = L.alloc_forward(dbf, dev, gather=args.gather)
        L.forward(dbf, bb, fb)
        torch.cuda.synchronize()
        ref = fb["out"].double()
        err = ((bufs[0]["out"].double() - ref).abs().max() /
               ref.abs().max()).item()
        line["mxfp8_error"] = {
            "max_rel_err_vs_bf16_layer": round(err, 5),
            "what": "max|out_mxfp8 - out_bf16| / max|out_bf16| over the "
                    "whole output of batch 0"}
        del fb
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, base, bufs[0]["logits"],
                                            min(args.cpu_tokens, cfg.T))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
