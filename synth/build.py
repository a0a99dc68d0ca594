"""Build the synthetic-input generator libraries in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops stay disabled in every HIP build of this repository.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout
                           + r.stderr)


def build_host():
    out = os.path.join(HERE, "libsynth_host.so")
    _run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-o", out, "synth_host.c"])
    return out


def build_dev():
    out = os.path.join(HERE, "libsynth_dev.so")
    _run([HIPCC] + HIP_FLAGS + ["-o", out, "synth_dev.hip"])
    return out


def build():
    return build_host(), build_dev()


if __name__ == "__main__":
    print(build())
