"""Bounds checking of the host code: csrc/api.cpp's argument validation
and workspace sizing built with AddressSanitizer (host pass only; the
device code is unchanged) and driven by tests/host/api_asan_check.cpp,
which hands every struct over heap-allocated at its exact size and calls
each entry point with arguments it must reject before any device work,
plus 20000 random descriptors through the workspace-size queries. The
kernel launchers come from the built library."""
import os
import shutil
import subprocess

import pytest

from ragged_grouped_gemm_router_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ragged_grouped_gemm_router_amd")


def test_api_validation_under_asan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(B.OUT):
        pytest.skip("g++ or the built library is missing")
    obj = tmp_path / "api_asan.o"
    cmd = [B.hipcc(), *B.FLAGS, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fno-omit-frame-pointer", "-c",
           os.path.join(B.CSRC, "api.cpp"), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    drv = tmp_path / "drv.o"
    r = subprocess.run([gxx, "-std=c++17", "-g", "-O1", "-fsanitize=address",
                        "-c", os.path.join(ROOT, "tests", "host", "api_asan_check.cpp"),
                        "-o", str(drv)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "api_asan_check"
    rocm_lib = "/opt/rocm/lib"
    r = subprocess.run([gxx, "-fsanitize=address", str(obj), str(drv),
                        "-L" + PKG, "-lmoe_mi355x", "-Wl,-rpath," + PKG,
                        "-L" + rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib,
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=env)
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.stdout[-2000:] +
                                                             r.stderr[-4000:])
