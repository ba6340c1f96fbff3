"""Build libselscan.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("selscan_fwd.hip", "selscan_bwd.hip", "selscan_conv.hip")]
OUT = os.path.join(PKG, "libselscan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def build(extra=None, out=OUT, srcs=None, verbose=False) -> str:
    cmd = [HIPCC, *HIP_FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out,
           *(srcs or SRCS)]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
