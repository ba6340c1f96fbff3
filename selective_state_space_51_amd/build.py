"""Build libselscan.so in-tree with hipcc for gfx950 (cross-compiles without a GPU), and beside it
two diagnostic libraries: libselscan_ubench.so (the microbenchmarks) and libselscan_phases.so (the
scan library with the backward's per-wave phase clocks compiled in).  The sources compile in
parallel to objects in a temporary directory, then link."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("selscan_fwd.hip", "selscan_bwd.hip", "selscan_conv.hip")]
OUT = os.path.join(PKG, "libselscan.so")
UBENCH_SRCS = [os.path.join(CSRC, "ubench.hip")]
UBENCH_OUT = os.path.join(PKG, "libselscan_ubench.so")
PHASES_OUT = os.path.join(PKG, "libselscan_phases.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)


def build(extra=None, out=OUT, srcs=None, verbose=False) -> str:
    """Compile `srcs` (default: the scan library's sources) and link them into the shared object
    `out`; `extra` flags go to every hipcc line."""
    srcs = srcs or SRCS
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="selscan_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
            futs = [ex.submit(_run, [HIPCC, *HIP_FLAGS, *(extra or []), *inc, "-c", "-o", o, s], verbose)
                    for s, o in zip(srcs, objs)]
            for f in futs:
                f.result()
        tmp_out = out + ".tmp"
        _run([HIPCC, *HIP_FLAGS, *(extra or []), "-shared", "-o", tmp_out, *objs], verbose)
        os.replace(tmp_out, out)
    return out


def build_all(extra=None, verbose=False) -> None:
    """The scan library and the two diagnostic libraries, compiled side by side."""
    with cf.ThreadPoolExecutor(max_workers=3) as ex:
        futs = [ex.submit(build, extra, OUT, SRCS, verbose),
                ex.submit(build, extra, UBENCH_OUT, UBENCH_SRCS, verbose),
                ex.submit(build, [*(extra or []), "-DSELSCAN_PHASE_CLOCKS"], PHASES_OUT, SRCS, verbose)]
        for f in futs:
            f.result()


if __name__ == "__main__":
    build_all(extra=sys.argv[1:], verbose=True)
