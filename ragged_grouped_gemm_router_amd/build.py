"""Build the C-ABI library libmoe_mi355x.so for gfx950 with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, into objects under _build/, then linked into a shared
library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe_mi355x.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.cpp", "route.hip", "perm.hip", "gemm_simt.hip",
           "gemm_mfma.hip", "mxfp8.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = OUT, extra_flags=()) -> str:
    """Compile every source and link ``out``. ``extra_flags`` (e.g. -D
    switches of kernel variants) go to every hipcc compile."""
    build_dir = BUILD if out == OUT else os.path.join(
        BUILD, "variant_" + os.path.basename(os.path.dirname(out)))
    os.makedirs(build_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, list(extra_flags)),
                           srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    # python build.py [OUT_SO -DFLAG ...]
    if len(sys.argv) > 1:
        build(verbose=True, out=os.path.abspath(sys.argv[1]),
              extra_flags=sys.argv[2:])
    else:
        build(verbose=True)
    sys.exit(0)
