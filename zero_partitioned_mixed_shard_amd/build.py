"""Build libzero_shard.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# owner-step kernels + C ABI, and the flat copy kernels; zero_common.h is
# included by both
SRCS = [os.path.join(PKG, "csrc", f) for f in ("zero_shard.hip", "zero_flat.hip")]
LIB = os.path.join(PKG, "libzero_shard.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # one IEEE rounding per operation, on host and device alike
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra=()) -> str:
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, *FLAGS, *extra, "-o", tmp, *SRCS], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
