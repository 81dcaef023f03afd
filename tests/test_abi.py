"""The C-ABI library loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before touching the GPU. CPU only:
every call here fails validation, so no HIP work is ever enqueued."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from ragged_grouped_gemm_router_amd import binding as B
from ragged_grouped_gemm_router_amd import layer as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_named_calls():
    fns = declared_functions()
    for name in ("moe_route", "moe_permute", "moe_grouped_gemm_swiglu",
                 "moe_unpermute_combine", "moe_forward", "moe_backward"):
        assert name in fns
    assert set(fns) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_struct_layouts_match_header():
    # int32 x 10; six pointers; pointer-only argument blocks
    assert ctypes.sizeof(B.MoeDesc) == 40
    assert ctypes.sizeof(B.MoeExpertWeights) == 48
    n_ptr_fwd = 4 + 1 + 14 + B.MOE_FWD_NEVENTS
    assert ctypes.sizeof(B.MoeFwdArgs) == 8 * n_ptr_fwd + 2 * 48
    n_ptr_bwd = 2 + 18 + 5 + 4 + B.MOE_BWD_NEVENTS
    assert ctypes.sizeof(B.MoeBwdArgs) == 8 * n_ptr_bwd + 2 * 48


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_str(s).startswith(b"MOE_")
    assert b"unknown" in lib.moe_status_str(99)


def _ws(desc, bwd=False):
    return B.moe_workspace_size(desc, bwd)


def test_workspace_size_host_only():
    d = B.make_desc(4096, 7168, 2048, 256, 8, 2048, "sigmoid")
    n = _ws(d)
    assert n >= 4 * 256 * 32 + 2 * 4096 * 2048  # histogram + shared hidden
    nb = _ws(d.__class__(4096, 7168, 2048, 256, 8, 0, 1, 1, 1, 0), True)
    assert nb >= 2 * 32768 * (2 * 7168 + 2 * 2048)


def test_flags_accepted():
    """Every defined flag bit is a valid descriptor."""
    d = B.make_desc(64, 128, 256, 8, 2)
    for fl in (B.MOE_FLAG_SAVE_ACTS, B.MOE_FLAG_NO_TAIL_SPLIT,
               B.MOE_FLAG_SAVE_ACTS | B.MOE_FLAG_NO_TAIL_SPLIT):
        d.flags = fl
        assert _ws(d) > 0


@pytest.mark.parametrize("fields,code", [
    (dict(K=3, E=2), B.MOE_EINVAL),              # K > E
    (dict(K=0), B.MOE_EINVAL),
    (dict(T=-1), B.MOE_EINVAL),
    (dict(E=2000, K=2), B.MOE_EUNSUPPORTED),     # E > E_MAX
    (dict(K=17, E=64), B.MOE_EUNSUPPORTED),      # K > K_MAX
    (dict(d_model=100), B.MOE_EUNSUPPORTED),     # not a multiple of 8
    (dict(gate=7), B.MOE_EINVAL),
    (dict(act_dtype=5), B.MOE_EINVAL),
    (dict(flags=8), B.MOE_EINVAL),
    (dict(flags=4), B.MOE_EINVAL),               # no such flag
    (dict(gemm_dtype=B.MOE_F32), B.MOE_EINVAL),             # bf16 act, f32 gemm
    (dict(gemm_dtype=B.MOE_MXFP8, d_model=160), B.MOE_EUNSUPPORTED),
    (dict(gemm_dtype=B.MOE_MXFP8, d_ff_shared=96), B.MOE_EUNSUPPORTED),
    (dict(gemm_dtype=B.MOE_MXFP8, act_dtype=B.MOE_F32), B.MOE_EINVAL),
])
def test_bad_descriptor(fields, code):
    d = B.make_desc(64, 128, 256, 8, 2)
    for k, v in fields.items():
        setattr(d, k, v)
    n = ctypes.c_size_t(0)
    assert B.load().moe_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == code
    fake = 0x1000
    assert B.load().moe_route(ctypes.byref(d), fake, fake, None, None, fake,
                              fake, fake, None) == code


def test_null_pointers_rejected():
    lib = B.load()
    d = B.make_desc(64, 128, 256, 8, 2)
    fake = 0x1000
    # missing topk outputs
    assert lib.moe_route(ctypes.byref(d), fake, fake, None, None, fake, None,
                         fake, None) == B.MOE_EINVAL
    # router needed but no logits_out
    assert lib.moe_route(ctypes.byref(d), fake, fake, None, None, None, fake,
                         fake, None) == B.MOE_EINVAL
    assert lib.moe_unpermute_combine(ctypes.byref(d), None, fake, fake, None,
                                     fake, None) == B.MOE_EINVAL
    assert lib.moe_route(None, fake, fake, None, None, fake, fake, fake,
                         None) == B.MOE_EINVAL


def test_workspace_too_small_rejected():
    lib = B.load()
    d = B.make_desc(64, 128, 256, 8, 2)
    fake = 0x1000
    st = lib.moe_permute(ctypes.byref(d), fake, fake, fake, fake, fake, fake,
                         fake, None, fake, 16, None)
    assert st == B.MOE_EWORKSPACE
    a = B.MoeFwdArgs()
    for name in ("x", "w_router", "out", "logits", "topk_idx", "topk_w",
                 "counts", "offsets", "sorted_src", "dest", "x_perm", "h",
                 "y_perm"):
        setattr(a, name, fake)
    a.routed = B.MoeExpertWeights(fake, fake, fake, None, None, None)
    assert lib.moe_forward(ctypes.byref(d), ctypes.byref(a), fake, 16,
                           None) == B.MOE_EWORKSPACE
    a.h = None
    assert lib.moe_forward(ctypes.byref(d), ctypes.byref(a), fake, 1 << 30,
                           None) == B.MOE_EINVAL


def test_save_acts_requires_buffers():
    lib = B.load()
    d = B.make_desc(64, 128, 256, 8, 2, save_acts=True)
    fake = 0x1000
    w = B.MoeExpertWeights(fake, fake, fake, None, None, None)
    st = lib.moe_grouped_gemm_swiglu(ctypes.byref(d), fake, None, fake,
                                     ctypes.byref(w), None, ctypes.byref(w),
                                     fake, fake, None, None, None, fake,
                                     1 << 30, None)
    assert st == B.MOE_EINVAL


def test_router_backward_validation():
    lib = B.load()
    d = B.make_desc(64, 128, 256, 8, 2)
    fake = 0x1000
    n = ctypes.c_size_t(0)
    assert lib.moe_router_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_OK
    assert n.value >= 64 * 128 * 2  # the router's share of dx

    def call(desc, ws_bytes=n.value, aux_coef=0.0, **null):
        names = ["x", "w_router", "logits", "topk_idx", "topk_w", "d_topk_w",
                 "counts"]
        head = [None if k in null else fake for k in names]
        tail = [None if k in null else fake
                for k in ("d_logits", "d_w_router", "dx", "ws")]
        return lib.moe_router_backward(ctypes.byref(desc), *head, aux_coef,
                                       *tail, ws_bytes, None)

    assert call(d, d_topk_w=1) == B.MOE_EINVAL
    assert call(d, ws_bytes=16) == B.MOE_EWORKSPACE
    # counts may be NULL only without the balance loss
    assert call(d, aux_coef=0.01, counts=1) == B.MOE_EINVAL
    assert call(d, aux_coef=float("nan")) == B.MOE_EINVAL
    z = B.make_desc(0, 128, 256, 8, 2)
    assert lib.moe_router_backward(ctypes.byref(z), *([None] * 7), 0.0,
                                   *([None] * 4), 0, None) == B.MOE_OK


def test_balance_stats_validation():
    lib = B.load()
    d = B.make_desc(64, 128, 256, 8, 2)
    fake = 0x1000
    n = ctypes.c_size_t(0)
    assert lib.moe_router_workspace_size(ctypes.byref(d), ctypes.byref(n)) == B.MOE_OK
    ok = [fake] * 6
    for i in range(6):
        bad = list(ok)
        bad[i] = None
        assert lib.moe_load_balance_stats(ctypes.byref(d), *bad, n.value,
                                          None) == B.MOE_EINVAL
    assert lib.moe_load_balance_stats(ctypes.byref(d), *ok, 16,
                                      None) == B.MOE_EWORKSPACE
    z = B.make_desc(0, 128, 256, 8, 2)
    assert lib.moe_load_balance_stats(ctypes.byref(z), *([None] * 6), 0,
                                      None) == B.MOE_OK

def test_bias_update_and_monitor_validation():
    lib = B.load()
    d = B.make_desc(64, 128, 256, 8, 2)
    fake = 0x1000
    upd = lib.moe_update_route_bias
    assert upd(ctypes.byref(d), None, fake, 0.01, 0.0, 0, None, None) == B.MOE_EINVAL
    assert upd(ctypes.byref(d), fake, None, 0.01, 0.0, 0, None, None) == B.MOE_EINVAL
    assert upd(ctypes.byref(d), fake, fake, 0.01, 0.0, 2, None, None) == B.MOE_EINVAL
    assert upd(ctypes.byref(d), fake, fake, float("nan"), 0.0, 0, None,
               None) == B.MOE_EINVAL
    z = B.make_desc(0, 128, 256, 8, 2)
    assert upd(ctypes.byref(z), fake, fake, 0.01, 0.0, 1, None, None) == B.MOE_OK
    mon = lib.moe_balance_monitor
    assert mon(ctypes.byref(d), fake, 0, fake, None) == B.MOE_EINVAL
    assert mon(ctypes.byref(d), None, 4, fake, None) == B.MOE_EINVAL
    assert mon(ctypes.byref(d), fake, 4, None, None) == B.MOE_EINVAL


def test_mxfp8_backward_validation():
    lib = B.load()
    fake = 0x1000
    d = B.make_desc(64, 128, 256, 8, 2, mxfp8=True)
    nb = _ws(d, True)
    a = B.MoeBwdArgs()
    for k in ("dy", "x", "topk_idx", "topk_w", "offsets", "sorted_src", "dest",
              "x_perm", "h", "y_perm", "dx", "dw1", "dw3", "dw2", "d_topk_w",
              "x_perm_scales", "w2t", "w2t_scales", "w13t", "w13t_scales"):
        setattr(a, k, fake)
    a.routed = B.MoeExpertWeights(fake, fake, fake, fake, fake, fake)
    assert lib.moe_backward(ctypes.byref(d), ctypes.byref(a), fake, 16,
                            None) == B.MOE_EWORKSPACE
    a.w13t = None
    assert lib.moe_backward(ctypes.byref(d), ctypes.byref(a), fake, nb,
                            None) == B.MOE_EINVAL
    a.w13t = fake
    a.act_a = fake  # saved pre-activations come in pairs
    assert lib.moe_backward(ctypes.byref(d), ctypes.byref(a), fake, nb,
                            None) == B.MOE_EINVAL
    a.act_a = None
    # a shared expert needs its MX weights and transposed copies
    ds = B.make_desc(64, 128, 256, 8, 2, d_ff_shared=128, mxfp8=True)
    assert lib.moe_backward(ctypes.byref(ds), ctypes.byref(a), fake,
                            _ws(ds, True), None) == B.MOE_EINVAL
    assert _ws(ds, True) > nb
    # the MX backward's workspace holds the quantised dy_perm [T*K, d] and
    # [da | db] [T*K, 2 f] besides the bf16 buffers
    TK, d, f = 128, 128, 256
    assert nb > 2 * TK * (2 * d + 2 * f) + TK * d + TK * 2 * f


def test_quantize_t_validation():
    lib = B.load()
    fake = 0x1000
    q = lib.moe_quantize_mxfp8_t
    assert q(None, 2, 64, 128, fake, fake, 64, 0, None) == B.MOE_EINVAL
    assert q(fake, 2, 64, 128, fake, fake, 96, 64, None) == B.MOE_EINVAL
    assert q(fake, 2, 48, 128, fake, fake, 64, 0, None) == B.MOE_EUNSUPPORTED
    assert q(fake, 2, 64, 96, fake, fake, 64, 0, None) == B.MOE_EUNSUPPORTED
    assert q(fake, 0, 64, 128, None, None, 64, 0, None) == B.MOE_OK
    assert q(fake, -1, 64, 128, fake, fake, 64, 0, None) == B.MOE_EINVAL
    # the destination's 128-column scale spans: ldq and col_off multiples
    # of 128
    assert q(fake, 2, 64, 128, fake, fake, 192, 64, None) == B.MOE_EUNSUPPORTED
    assert q(fake, 2, 64, 128, fake, fake, 96, 0, None) == B.MOE_EUNSUPPORTED


def test_quantize_validation():
    lib = B.load()
    fake = 0x1000
    q = lib.moe_quantize_mxfp8
    assert q(None, 4, 128, fake, fake, None) == B.MOE_EINVAL
    assert q(fake, 4, 0, fake, fake, None) == B.MOE_EINVAL
    assert q(fake, 4, 96, fake, fake, None) == B.MOE_EUNSUPPORTED
    assert q(fake, 0, 128, fake, fake, None) == B.MOE_OK
    # scale arrays are written a 4-code word at a time
    assert q(fake, 4, 128, fake, fake + 2, None) == B.MOE_EINVAL
    qt = lib.moe_quantize_mxfp8_t
    assert qt(fake, 2, 64, 128, fake, fake + 1, 128, 0, None) == B.MOE_EINVAL


def test_mx_scale_layout_views():
    """The scale arrays' layout: the code of block b of row r of an
    R-row operand at byte ((b // 4) * R + r) * 4 + b % 4; the Python
    views take it to rows of cols / 32 codes and back."""
    R, cols = 5, 384
    flat = torch.arange(R * cols // 32, dtype=torch.int64)
    sc = flat.reshape(L.mx_scale_shape(R, cols))
    rows = L.mx_scales_rows(sc, (R,))
    for r in range(R):
        for b in range(cols // 32):
            assert rows[r, b] == ((b // 4) * R + r) * 4 + b % 4
    # stacked batches: row r of operand e is row e * R + r
    E = 3
    sc = torch.arange(E * R * cols // 32).reshape(L.mx_scale_shape(E * R, cols))
    per = L.mx_scales_rows(sc, (E, R))
    assert per[2, 1, 5] == ((5 // 4) * E * R + 2 * R + 1) * 4 + 5 % 4


def test_bf16_backward_workspace_exact():
    """The bf16 backward (no shared expert) keeps only the tile prefixes of
    the four row-tile heights and dy_perm, da, db and dx_perm, each block
    aligned to 256 bytes: the data and weight gradients read the weights
    and activations as stored, with no transposed copies."""
    def al(n):
        return (n + 255) // 256 * 256
    for T, dm, f, E, K in ((2048, 128, 192, 8, 2), (4096, 7168, 2048, 256, 8)):
        d = B.make_desc(T, dm, f, E, K)
        TK = T * K
        want = (4 * al(4 * (E + 1)) + 2 * al(2 * TK * dm) +
                2 * al(2 * TK * f))
        assert _ws(d, True) == want, (T, dm, f, E, K)
