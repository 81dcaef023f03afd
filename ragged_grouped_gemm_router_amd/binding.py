"""ctypes binding of libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: torch tensors supply device memory and
torch's current stream supplies the HIP stream; every step of the layer
runs in the library's HIP kernels. If the library is not built the
binding raises; there is no other implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p, POINTER
from typing import Optional

import torch

# MOE_LIB_PATH selects another build of the same library (kernel variants
# built with different compile-time switches, for A/B measurements).
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID = 0, 1
MOE_FLAG_SAVE_ACTS = 1
MOE_FLAG_NO_TAIL_SPLIT = 2
MOE_K_MAX, MOE_E_MAX = 16, 1024
MOE_FWD_NEVENTS, MOE_BWD_NEVENTS = 6, 8
MOE_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTED = ["moe_status_str", "moe_workspace_size", "moe_route",
            "moe_permute", "moe_grouped_gemm_swiglu", "moe_unpermute_combine",
            "moe_forward", "moe_backward", "moe_router_workspace_size",
            "moe_router_backward", "moe_load_balance_stats",
            "moe_update_route_bias", "moe_balance_monitor",
            "moe_quantize_mxfp8", "moe_quantize_mxfp8_t",
            "moe_forward_noalloc"]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "T", "d_model", "d_ff", "E", "K", "d_ff_shared", "gate", "act_dtype",
        "gemm_dtype", "flags")]


class MoeExpertWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "w1", "w3", "w2", "w1_scales", "w3_scales", "w2_scales")]


class MoeFwdArgs(ctypes.Structure):
    _fields_ = [
        ("x", c_void_p), ("w_router", c_void_p), ("route_bias", c_void_p),
        ("logits_in", c_void_p), ("routed", MoeExpertWeights),
        ("shared", MoeExpertWeights), ("out", c_void_p), ("logits", c_void_p),
        ("topk_idx", c_void_p), ("topk_w", c_void_p), ("counts", c_void_p),
        ("offsets", c_void_p), ("sorted_src", c_void_p), ("dest", c_void_p),
        ("x_perm", c_void_p), ("x_perm_scales", c_void_p), ("h", c_void_p),
        ("y_perm", c_void_p), ("y_shared", c_void_p), ("act_a", c_void_p),
        ("act_b", c_void_p), ("events", c_void_p * MOE_FWD_NEVENTS)]


class MoeBwdArgs(ctypes.Structure):
    _fields_ = [
        ("dy", c_void_p), ("x", c_void_p), ("routed", MoeExpertWeights),
        ("shared", MoeExpertWeights), ("topk_idx", c_void_p),
        ("topk_w", c_void_p), ("offsets", c_void_p), ("sorted_src", c_void_p),
        ("dest", c_void_p), ("x_perm", c_void_p), ("h", c_void_p),
        ("y_perm", c_void_p), ("act_a", c_void_p), ("act_b", c_void_p),
        ("dx", c_void_p), ("dw1", c_void_p), ("dw3", c_void_p),
        ("dw2", c_void_p), ("d_topk_w", c_void_p),
        ("dws1", c_void_p), ("dws3", c_void_p), ("dws2", c_void_p),
        ("x_perm_scales", c_void_p), ("w2t", c_void_p),
        ("w2t_scales", c_void_p), ("w13t", c_void_p),
        ("w13t_scales", c_void_p), ("ws2t", c_void_p),
        ("ws2t_scales", c_void_p), ("ws13t", c_void_p),
        ("ws13t_scales", c_void_p),
        ("events", c_void_p * MOE_BWD_NEVENTS)]


_LIB = None


def load() -> ctypes.CDLL:
    """Load the built library and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "ragged_grouped_gemm_router_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    D = POINTER(MoeDesc)
    sig = {
        "moe_status_str": (ctypes.c_char_p, [c_int32]),
        "moe_workspace_size": (c_int32, [D, c_int32, POINTER(c_size_t)]),
        "moe_route": (c_int32, [D] + [c_void_p] * 8),
        "moe_permute": (c_int32, [D] + [c_void_p] * 9 + [c_size_t, c_void_p]),
        "moe_grouped_gemm_swiglu": (c_int32, [
            D, c_void_p, c_void_p, c_void_p, POINTER(MoeExpertWeights),
            c_void_p, POINTER(MoeExpertWeights), c_void_p, c_void_p,
            c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_unpermute_combine": (c_int32, [D] + [c_void_p] * 6),
        "moe_forward": (c_int32, [D, POINTER(MoeFwdArgs), c_void_p, c_size_t,
                                  c_void_p]),
        "moe_forward_noalloc": (c_int32, [D, POINTER(MoeFwdArgs), c_void_p]),
        "moe_backward": (c_int32, [D, POINTER(MoeBwdArgs), c_void_p,
                                   c_size_t, c_void_p]),
        "moe_quantize_mxfp8_t": (c_int32, [c_void_p, c_int64, c_int64,
                                           c_int64, c_void_p, c_void_p,
                                           c_int64, c_int64, c_void_p]),
        "moe_quantize_mxfp8": (c_int32, [c_void_p, c_int64, c_int64,
                                         c_void_p, c_void_p, c_void_p]),
        "moe_router_workspace_size": (c_int32, [D, POINTER(c_size_t)]),
        "moe_router_backward": (c_int32, [D] + [c_void_p] * 7 + [c_float] +
                                [c_void_p] * 4 + [c_size_t, c_void_p]),
        "moe_load_balance_stats": (c_int32, [D] + [c_void_p] * 6 +
                                   [c_size_t, c_void_p]),
        "moe_update_route_bias": (c_int32, [D, c_void_p, c_void_p, c_float,
                                            c_float, c_int32, c_void_p,
                                            c_void_p]),
        "moe_balance_monitor": (c_int32, [D, c_void_p, c_int32, c_void_p,
                                          c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


# ----------------------------------------------------------------- helpers
def ptr(t: Optional[torch.Tensor]):
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def current_stream():
    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


def check(status: int, what: str):
    if status != MOE_OK:
        msg = load().moe_status_str(status).decode()
        raise MoeError(status, f"{what}: {msg}")


def make_desc(T: int, d_model: int, d_ff: int, E: int, K: int,
              d_ff_shared: int = 0, gate: str = "softmax",
              dtype: str = "bf16", mxfp8: bool = False,
              save_acts: bool = False) -> MoeDesc:
    act = MOE_F32 if dtype == "f32" else MOE_BF16
    return MoeDesc(T, d_model, d_ff, E, K, d_ff_shared,
                   MOE_GATE_SIGMOID if gate == "sigmoid" else MOE_GATE_SOFTMAX,
                   act, MOE_MXFP8 if mxfp8 else act,
                   MOE_FLAG_SAVE_ACTS if save_acts else 0)


def expert_weights(w1=None, w3=None, w2=None, s1=None, s3=None, s2=None):
    return MoeExpertWeights(ptr(w1), ptr(w3), ptr(w2), ptr(s1), ptr(s3),
                            ptr(s2))


# ------------------------------------------------------------ entry points
def moe_workspace_size(desc: MoeDesc, for_backward: bool = False) -> int:
    n = c_size_t(0)
    check(load().moe_workspace_size(ctypes.byref(desc), int(for_backward),
                                    ctypes.byref(n)), "moe_workspace_size")
    return n.value


def moe_route(desc, x, w_router, route_bias, logits_in, logits_out,
              topk_idx, topk_w, stream=None):
    check(load().moe_route(ctypes.byref(desc), ptr(x), ptr(w_router),
                           ptr(route_bias), ptr(logits_in), ptr(logits_out),
                           ptr(topk_idx), ptr(topk_w),
                           stream if stream is not None else current_stream()),
          "moe_route")


def moe_permute(desc, x, topk_idx, counts, offsets, sorted_src, dest, x_perm,
                x_perm_scales, ws, stream=None):
    check(load().moe_permute(ctypes.byref(desc), ptr(x), ptr(topk_idx),
                             ptr(counts), ptr(offsets), ptr(sorted_src),
                             ptr(dest), ptr(x_perm), ptr(x_perm_scales),
                             ptr(ws), ws.numel() * ws.element_size(),
                             stream if stream is not None else current_stream()),
          "moe_permute")


def moe_grouped_gemm_swiglu(desc, x_perm, x_perm_scales, offsets, routed,
                            x_shared, shared, h, y_perm, y_shared, act_a,
                            act_b, ws, stream=None):
    check(load().moe_grouped_gemm_swiglu(
        ctypes.byref(desc), ptr(x_perm), ptr(x_perm_scales), ptr(offsets),
        ctypes.byref(routed), ptr(x_shared),
        ctypes.byref(shared if shared is not None else MoeExpertWeights()),
        ptr(h), ptr(y_perm), ptr(y_shared), ptr(act_a), ptr(act_b), ptr(ws),
        ws.numel() * ws.element_size(),
        stream if stream is not None else current_stream()),
        "moe_grouped_gemm_swiglu")


def moe_unpermute_combine(desc, y_perm, dest, topk_w, y_shared, out,
                          stream=None):
    check(load().moe_unpermute_combine(
        ctypes.byref(desc), ptr(y_perm), ptr(dest), ptr(topk_w),
        ptr(y_shared), ptr(out),
        stream if stream is not None else current_stream()),
        "moe_unpermute_combine")


def moe_forward(desc, args: MoeFwdArgs, ws, stream=None):
    check(load().moe_forward(ctypes.byref(desc), ctypes.byref(args), ptr(ws),
                             ws.numel() * ws.element_size(),
                             stream if stream is not None else current_stream()),
          "moe_forward")


def moe_forward_noalloc(desc, args: MoeFwdArgs, stream=None):
    check(load().moe_forward_noalloc(
        ctypes.byref(desc), ctypes.byref(args),
        stream if stream is not None else current_stream()),
        "moe_forward_noalloc")


def moe_backward(desc, args: MoeBwdArgs, ws, stream=None):
    check(load().moe_backward(ctypes.byref(desc), ctypes.byref(args), ptr(ws),
                              ws.numel() * ws.element_size(),
                              stream if stream is not None else current_stream()),
          "moe_backward")


def moe_router_workspace_size(desc: MoeDesc) -> int:
    n = c_size_t(0)
    check(load().moe_router_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
          "moe_router_workspace_size")
    return n.value


def moe_router_backward(desc, x, w_router, logits, topk_idx, topk_w,
                        d_topk_w, counts, aux_coef, d_logits, d_w_router, dx,
                        ws, stream=None):
    check(load().moe_router_backward(
        ctypes.byref(desc), ptr(x), ptr(w_router), ptr(logits), ptr(topk_idx),
        ptr(topk_w), ptr(d_topk_w), ptr(counts), float(aux_coef),
        ptr(d_logits), ptr(d_w_router), ptr(dx),
        ptr(ws), ws.numel() * ws.element_size(),
        stream if stream is not None else current_stream()),
        "moe_router_backward")


def moe_load_balance_stats(desc, logits, counts, f, p_mean, aux, ws,
                           stream=None):
    check(load().moe_load_balance_stats(
        ctypes.byref(desc), ptr(logits), ptr(counts), ptr(f), ptr(p_mean),
        ptr(aux), ptr(ws), ws.numel() * ws.element_size(),
        stream if stream is not None else current_stream()),
        "moe_load_balance_stats")


def moe_update_route_bias(desc, counts, route_bias, gamma, target=0.0,
                          rule=0, load_out=None, stream=None):
    check(load().moe_update_route_bias(
        ctypes.byref(desc), ptr(counts), ptr(route_bias), float(gamma),
        float(target), int(rule), ptr(load_out),
        stream if stream is not None else current_stream()),
        "moe_update_route_bias")


def moe_balance_monitor(desc, load_hist, out, stream=None):
    check(load().moe_balance_monitor(
        ctypes.byref(desc), ptr(load_hist), int(load_hist.shape[0]), ptr(out),
        stream if stream is not None else current_stream()),
        "moe_balance_monitor")


def moe_quantize_mxfp8(src, rows, cols, q, scales, stream=None):
    check(load().moe_quantize_mxfp8(
        ptr(src), rows, cols, ptr(q), ptr(scales),
        stream if stream is not None else current_stream()),
        "moe_quantize_mxfp8")


def moe_quantize_mxfp8_t(src, batch, rows, cols, q, scales, ldq, col_off=0,
                         stream=None):
    check(load().moe_quantize_mxfp8_t(
        ptr(src), batch, rows, cols, ptr(q), ptr(scales), ldq, col_off,
        stream if stream is not None else current_stream()),
        "moe_quantize_mxfp8_t")
