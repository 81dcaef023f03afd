"""Dropless MoE expert layer for AMD MI355X (gfx950): router, top-K gate,
stable permutation, ragged grouped SwiGLU GEMMs on MFMA, combine, backward
and an MXFP8 forward, as hand-written HIP kernels behind a C ABI
(include/moe.h). This package holds the kernels' sources (csrc/), the
build script and a thin ctypes binding."""
from . import accounting  # noqa: F401
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MoeError, make_desc, moe_backward, moe_forward, moe_grouped_gemm_swiglu,
    moe_permute, moe_quantize_mxfp8, moe_route, moe_unpermute_combine,
    moe_workspace_size,
)
