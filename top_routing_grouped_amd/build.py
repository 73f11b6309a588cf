"""Build libmoe.so (gfx950) in-tree with hipcc.

    python -m top_routing_grouped_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, and linked with the C ABI layer into
top_routing_grouped_amd/libmoe.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero"]

# Per-source device options.  The MFMA issue-rate loop keeps its accumulators
# in ordinary VGPRs: with the default accumulator-register form the compiler
# copies some 16x16 accumulators between register files on every iteration,
# and the loop then times those copies instead of the matrix cores.
EXTRA_DEVICE = {"moe_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

SOURCES = ["moe_gemm.hip", "moe_gemm_tiled.hip", "moe_route.hip", "moe_permute.hip", "moe_down_combine.hip",
           "moe_norm.hip", "moe_stream.hip", "moe_api.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, *EXTRA_DEVICE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
