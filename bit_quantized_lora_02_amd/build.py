"""Build the gfx950 HIP library ``libqlora.so`` in-tree with hipcc.

Usage: ``python -m bit_quantized_lora_02_amd.build`` (or ``__graft_entry__.build()``).
The library is compiled for gfx950 only; it links the HIP runtime and nothing else.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqlora.so")
SOURCES = ["abi.hip", "quant.hip", "nf4_gemm.hip", "nf4_gemv.hip", "lora_gemm.hip", "adamw.hip", "merge.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed binary32 instructions stay off (they are not needed by these kernels)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every a * b + c written in the sources is two rounded operations (HIP's default would fuse
    # them into one FMA, and __fmul_rn / __fadd_rn are plain * and + in this toolchain); an FMA
    # is written as fmaf where one is meant
    "-ffp-contract=off",
    "-Wall",
    "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libqlora.so next to this file."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed building libqlora.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
