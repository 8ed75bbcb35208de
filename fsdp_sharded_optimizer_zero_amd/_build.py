"""Build libzero_shard.so (the C-ABI library) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzero_shard.so")
BENCH_LIB = os.path.join(PKG, "libzs_benchcopy.so")
# The same library built with at most 65,536 threads per launch and the
# step's streaming loads at every size: a test build that runs the
# multi-launch path of every entry point, and the streaming step, on small
# shards.
SMALLGRID_LIB = os.path.join(PKG, "libzero_shard_smallgrid.so")
SMALLGRID_THREADS = 65536
SMALLGRID_DEFS = [f"-DZS_MAX_LAUNCH_THREADS={SMALLGRID_THREADS}", "-DZS_STEP_STREAM_BYTES=0"]

# -ffp-contract=off: the step is defined with one rounding per operation.
# -packed-fp32-ops off: no v_pk_* fp32 instructions are generated.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
              "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "zs_host.o")
    abi_o = os.path.join(BUILD, "zs_abi.o")
    kern_o = os.path.join(BUILD, "zs_kernels.o")
    _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "zs_host.cpp"), "-o", host_o], verbose)
    _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "zs_abi.cpp"), "-o", abi_o], verbose)
    _run(["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, "zs_kernels.hip"), "-o", kern_o],
         verbose)
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", host_o,
          abi_o, kern_o], verbose)
    os.replace(LIB + ".tmp", LIB)
    small_o = os.path.join(BUILD, "zs_kernels_smallgrid.o")
    _run(["hipcc", *HIP_FLAGS, *SMALLGRID_DEFS, "-c",
          os.path.join(CSRC, "zs_kernels.hip"), "-o", small_o], verbose)
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", SMALLGRID_LIB + ".tmp",
          host_o, abi_o, small_o], verbose)
    os.replace(SMALLGRID_LIB + ".tmp", SMALLGRID_LIB)
    # bench-only copy kernel (not part of the ABI)
    _run(["hipcc", *HIP_FLAGS, "-shared", "-o", BENCH_LIB + ".tmp",
          os.path.join(CSRC, "zs_bench_copy.hip")], verbose)
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    return LIB


def device_asm(out_path: str) -> None:
    """Write the gfx950 assembly of the kernels (for inspection)."""
    _run(["hipcc", *HIP_FLAGS, "--cuda-device-only", "-S", "-o", out_path,
          os.path.join(CSRC, "zs_kernels.hip")], True)


if __name__ == "__main__":
    build(verbose=True)
