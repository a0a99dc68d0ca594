"""Build the gfx950 MoE layer library (libmoe_wq.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_wq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["abi.cpp", "route.hip", "permute.hip", "quant.hip", "ffn.hip",
           "ffn_decode.hip", "ffn_bitplane.hip", "ffn_prefill.hip",
           "combine.hip", "alloc.hip", "cache.hip", "cache.cpp", "noalloc.hip", "retile.hip"]
# Packed fp32 VALU instructions stay disabled in every HIP build here.
# MFMA accumulators are allocated in ordinary VGPRs (not AGPRs): the kernels
# rescale and convert accumulators with VALU instructions, which would
# otherwise need a move to and from the AGPR file for every element.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wno-unused-result", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libmoe_wq build failed:\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
