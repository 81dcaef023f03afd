"""The grouped GEMM's device tile list, checked on the CPU: the integer
decode the kernels run (csrc/tile_map.h: the dense n-group-major tile
order, the XCD remap, the group lookup in the tile prefix, the split of a
partial last round into quarter tiles, the contraction-grouped tiles) is
compiled into a host program that enumerates every workgroup of every
launch form the library issues, for 1500 random expert-count vectors
(empty, tiny, tile-edge, skewed and half-tile groups), and requires every
(row, column) of every group's output to be covered exactly once by a tile
of that group."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_tile_list_covers_every_output_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "tile_map_check"
    src = os.path.join(ROOT, "tests", "host", "tile_map_check.cpp")
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2",
                        "-std=c++17", "-Wno-unused-command-line-argument",
                        src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe), "1500"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout[-2000:]
