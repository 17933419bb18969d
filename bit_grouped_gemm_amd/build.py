"""Ahead-of-time build of the HIP library (gfx950 only) with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libmoe.so")
SOURCES = ["moe_api.hip", "moe_kernels.hip", "moe_gemm_big.hip", "moe_tile.hip", "moe_diag.hip", "moe_router.hip"]
HEADERS = ["moe_device.h", "moe_launch.h", os.path.join("..", "..", "include", "moe.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 arithmetic stays off: only scalar fp32 VALU ops are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


DRIVER_SRC = "moe_bench_main.cpp"
DRIVER = os.path.join(BUILD, "moe_bench")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile libmoe.so in-tree (always recompiles), then the standalone C++
    driver moe_bench linked against it (a torch-free caller of the ABI, used
    for profiling)."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = LIB + ".tmp"
    _run([HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp], verbose)
    os.replace(tmp, LIB)
    tmp = DRIVER + ".tmp"
    _run([HIPCC, "-O2", "-std=c++17", "-Wall", os.path.join(CSRC, DRIVER_SRC), "-L" + BUILD, "-lmoe",
          "-Wl,-rpath,$ORIGIN", "-o", tmp], verbose)
    os.replace(tmp, DRIVER)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
