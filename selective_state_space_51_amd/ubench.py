"""Microbenchmarks of the gfx950 resources the scan's roofline argument rests on.

  python -m selective_state_space_51_amd.ubench [--iters N] [--read-gib G]

Prints a markdown summary: for each VALU instruction form the scan kernels use (fp32 FMA and
multiply, v_exp_f32, v_rcp_f32, an FMA with a scalar operand, a DPP add, the scan's 5:1 mix of
FMA-class operations and exp, dependent chains, and exp next to FMAs that do or do not read its
result), the issue cost in SIMD cycles per wave64 instruction at 1, 2 and 4 waves per SIMD, with the shader clock measured inside the kernels (s_memtime against the 100 MHz
s_memrealtime); then the HBM read and copy streams in GB/s.  The kernels are in
csrc/ubench.hip, built into libselscan_ubench.so by build.py.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libselscan_ubench.so")
KINDS = ["fma", "mul", "exp", "fma_sgpr", "dpp_add", "rcp", "mix_5fma_1exp", "fma_chain1", "fma_chain2", "exp_chain1",
         "exp_fma_1to5_independent", "exp_fma_1to5_exp_read_next", "exp_fma_1to3_independent",
         "exp_fma_1to19_independent", "permlane32_swap", "permlane16_swap"]
# wave-instructions per loop iteration of each form
PER_ITER = {"mix_5fma_1exp": 54, "exp_fma_1to5_independent": 48, "exp_fma_1to5_exp_read_next": 48,
            "exp_fma_1to3_independent": 32, "exp_fma_1to19_independent": 40}
N_CU = 256
REALTIME_HZ = 100e6  # s_memrealtime counts a constant 100 MHz clock


def _lib():
    import torch  # noqa: F401  (the library binds to torch's HIP runtime)
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built; run selective_state_space_51_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.ub_valu_launch.argtypes = [ci, ci, ci, vp, vp, vp]
    lib.ub_valu_launch.restype = ci
    lib.ub_read_launch.argtypes = [vp, i64, ci, vp, vp]
    lib.ub_read_launch.restype = ci
    lib.ub_copy_launch.argtypes = [vp, vp, i64, ci, vp]
    lib.ub_copy_launch.restype = ci
    return lib


def valu(lib, torch, kind: int, waves_per_simd: int, iters: int, reps: int = 3):
    """Best of `reps` launches: (ns per wave-instruction per SIMD, shader clock in MHz)."""
    blocks = N_CU * waves_per_simd  # a workgroup is 4 waves: one per SIMD of its compute unit
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream()
    per_wave = iters * PER_ITER.get(KINDS[kind], 8)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        rc = lib.ub_valu_launch(kind, blocks, iters, out.data_ptr(), st.data_ptr(), s.cuda_stream)
        b.record(s)
        torch.cuda.synchronize()
        if rc:
            raise RuntimeError(f"ub_valu_launch({KINDS[kind]}) returned {rc}")
        ms = a.elapsed_time(b)
        stamps = st.view(blocks, 4).cpu().numpy().astype("float64")
        clk = (stamps[:, 1] - stamps[:, 0]).sum() / ((stamps[:, 3] - stamps[:, 2]).sum() / REALTIME_HZ) / 1e6
        ns = ms * 1e6 / (waves_per_simd * per_wave)
        if best is None or ns < best[0]:
            best = (ns, clk)
    return best


def streams(lib, torch, gib: float):
    n16 = int(gib * (1 << 30)) // 16
    src = torch.ones(n16 * 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    blocks = N_CU * 8
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    res = {}
    for name, launch, nbytes in (
            ("read", lambda: lib.ub_read_launch(src.data_ptr(), n16, blocks, out.data_ptr(), s.cuda_stream), 16 * n16),
            ("copy", lambda: lib.ub_copy_launch(src.data_ptr(), dst.data_ptr(), n16, blocks, s.cuda_stream),
             32 * n16)):
        launch()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            rc = launch()
            b.record(s)
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"ub_{name}_launch returned {rc}")
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        res[name] = (nbytes / (best * 1e-3) / 1e9, best)
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=40000)
    ap.add_argument("--read-gib", type=float, default=2.0)
    args = ap.parse_args(argv)
    import torch
    assert torch.cuda.is_available(), "the microbenchmarks need a GPU"
    lib = _lib()
    print("| form | waves/SIMD | ns per wave-instruction per SIMD | shader clock (MHz, in-kernel) "
          "| SIMD cycles per wave-instruction |")
    print("|---|---|---|---|---|")
    for k, name in enumerate(KINDS):
        for wps in (1, 2, 4):
            iters = args.iters * 8 // PER_ITER.get(name, 8)
            ns, clk = valu(lib, torch, k, wps, iters)
            print(f"| {name} | {wps} | {ns:.3f} | {clk:.0f} | {ns * clk / 1e3:.2f} |", flush=True)
    res = streams(lib, torch, args.read_gib)
    print()
    print("| stream | bytes moved | best ms | GB/s |")
    print("|---|---|---|---|")
    for name, (gbs, ms) in res.items():
        moved = args.read_gib * (2 if name == "copy" else 1)
        print(f"| {name} | {moved:g} GiB | {ms:.3f} | {gbs:.0f} |", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
