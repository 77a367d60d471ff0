"""Build libmoe_rounds.so (gfx950) in-tree with hipcc, and the benchmark's
matrix-core calibration library libmoe_calibrate.so.

Every source is compiled for gfx950 only. Packed fp32 instructions are
disabled on the device side (-packed-fp32-ops); the host pass warns that it
does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(OUT_DIR, "libmoe_rounds.so")
CALIB_LIB = os.path.join(OUT_DIR, "libmoe_calibrate.so")
CALIB_SOURCE = "calibrate.hip"
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["route_plan.hip", "dispatch_combine.hip", "grouped_gemm.hip",
           "wgrad.hip", "backward.hip", "api.hip"]
HEADERS = ["device_common.hpp", "launch.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CXXFLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
            "-I", os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", os.path.join(HERE, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # a kernel whose host-side launch stub was not emitted leaves an
    # undefined symbol that only shows when the library is loaded
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp],
                         capture_output=True, text=True, check=True).stdout
    missing = [ln.split()[-1] for ln in und.splitlines()
               if "device_stub" in ln or "_ZN3moe" in ln]
    if missing:
        raise RuntimeError(f"{tmp}: undefined kernel symbols {missing}")
    os.replace(tmp, LIB)
    # the calibration kernel: a library of its own, outside the layer's ABI
    cobj = _compile(CALIB_SOURCE, verbose)
    ctmp = CALIB_LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", ctmp, cobj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(ctmp, CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
