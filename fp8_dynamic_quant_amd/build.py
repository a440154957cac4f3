"""Build libwq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in place.

Usage: python -m fp8_dynamic_quant_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwq.so")

SOURCES = ["wq_api.hip", "k_quant.hip", "k_decode.hip", "k_fused.hip", "k_gemm_i8.hip", "k_gemm_tile.hip", "k_gemm_big.hip", "k_fp8.hip", "k_fp8_decode.hip", "k_moe.hip", "k_seg_decode.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # exact arithmetic: no contraction of a*b+c into fma, correctly rounded div/sqrt
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # the packed-FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(os.path.dirname(PKG), "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libwq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
