"""Build libtqkv.so (HIP, gfx950) in-tree with hipcc.

All device code is compiled with -ffp-contract=off (the store's codes are
defined in binary32 without contraction; the verify kernel asks for FMA
explicitly where it wants one) and with packed-FP32 instructions disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libtqkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale touches
    # them with VALU ops, and AGPR-resident accumulators were copied out and
    # back on every loop iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(extra_flags=(), out=LIB) -> str:
    """Compile every HIP source into `out` (libtqkv.so next to this file by
    default; always rebuilds)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
