"""Where a scan kernel's time goes, phase by phase.

  python -m selective_state_space_51_amd.phases [--pass fwd|bwd] [--workload NAME] [--calls K]

Binds the package to libselscan_phases.so (the scan library built by build.py with per-wave phase
clocks compiled into the forward and backward kernels) in place of libselscan.so, runs K calls of
the forward (--pass fwd) or one forward keeping the chunk states and then K backward calls
(--pass bwd), and prints, from the last call, the mean over waves of the shader-clock cycles each
wave spent in each phase of its chunk loop, and the whole kernel.  Forward phases: staging (the
barrier before, the wait for the chunk's loads, their commit to LDS, the barrier after), the issue
of the gate's and the next chunk's loads, the prologue's arithmetic, state loop, the y tile's LDS
writes and the barrier after them, the output stores.  Backward phases: staging (the
chunk's loads and their commit to LDS, between the two barriers around it), prologue, state loop
(its compute, and the waits at its two barriers apart), output.  Inputs are the workload's seeded
synthetic tensors.  Run from the repository root.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
PHASES_LIB = os.path.join(_PKG, "libselscan_phases.so")
PHASES = {"fwd": ["staging", "issue of the gate's and the next chunk's loads", "prologue arithmetic", "state loop",
                  "y tile to LDS and the barrier after it", "output stores"],
          "bwd": ["staging", "prologue", "state loop, outside its barriers", "state loop, first barrier wait",
                  "state loop, second barrier wait", "output"]}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd"], default="bwd")
    ap.add_argument("--workload", default="mamba1p4b_layer_b2_L65536_D4096")
    ap.add_argument("--calls", type=int, default=3)
    args = ap.parse_args(argv)
    if not os.path.exists(PHASES_LIB):
        raise ImportError(f"{PHASES_LIB} not built; run selective_state_space_51_amd/build.py")
    import numpy as np
    import torch

    import selective_state_space_51_amd as S
    import workloads as W

    assert torch.cuda.is_available(), "the phase clocks need a GPU"
    lib = S.use_library(PHASES_LIB)
    w = W.by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    t = {k: up(v) for k, v in W.generate(w).items()}
    op = {"selscan": S.SELSCAN_OP_FWD, "bidir": S.SELSCAN_OP_BIDIR, "ss2d": S.SELSCAN_OP_SS2D,
          "local_ss2d": S.SELSCAN_OP_LOCAL_SS2D}[w.kind]
    io = S.SELSCAN_BF16 if w.dtype == "bf16" else S.SELSCAN_F32
    geo = dict(H=w.H, W=w.W, window=w.window)
    need = S.selscan_workspace_bytes(op, w.batch, w.seqlen, w.dim, w.dstate, io)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    stream = torch.cuda.current_stream()
    bwd = args.pass_ == "bwd"
    y = torch.empty_like(t["x"])
    if bwd:
        _, ck = S.selscan_scan_fwd(op, t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                   chunk_states=True, workspace=ws, stream=stream, **geo)
        dy = up(W.generate_cotangent(w.batch, w.seqlen, w.dim, w.dtype))
        bws = torch.empty(S.selscan_scan_bwd_workspace_bytes(op, w.batch, w.seqlen, w.dim, w.dstate, io),
                          dtype=torch.uint8, device=dev)
    read, clear = (lib.selscan_bwd_phase_read, lib.selscan_bwd_phase_clear) if bwd else \
        (lib.selscan_fwd_phase_read, lib.selscan_fwd_phase_clear)
    read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    read.restype = ctypes.c_int
    clear.restype = ctypes.c_int
    grads = None
    ms = 0.0
    for _ in range(args.calls):
        torch.cuda.synchronize()
        if clear() != 0:
            raise RuntimeError("clearing the phase record failed")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        if bwd:
            grads = S.selscan_scan_bwd(op, t["x"], t["delta"], t["A"], t["B"], t["C"], dy, ck, D=t["D"], z=t["z"],
                                       workspace=bws, stream=stream, grads=grads, **geo)
        else:
            S.selscan_scan_fwd(op, t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], y=y,
                               workspace=ws, stream=stream, **geo)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
    rec = np.zeros((1 << 14) * 8, dtype=np.uint64)
    rc = read(ctypes.c_void_p(rec.ctypes.data), ctypes.c_size_t(rec.size))
    if rc != 0:
        raise RuntimeError(f"reading the phase record returned {rc}")
    rec = rec.reshape(-1, 8)
    rec = rec[rec[:, 7] == 1].astype(np.float64)
    total = rec[:, 6].mean()
    names = PHASES[args.pass_]
    print(f"workload {w.name}: {'backward' if bwd else 'forward'}, {rec.shape[0]} waves; cycles per wave "
          "(shader clock), mean over waves")
    print(f"last call: {ms:.3f} ms for all its launches (the phase-clocked scan kernel"
          f"{' and the reduction' if bwd else ''})")
    print()
    print("| phase | cycles per wave | share of the kernel |")
    print("|---|---|---|")
    for i, name in enumerate(names):
        print(f"| {name} | {rec[:, i].mean():.4g} | {100 * rec[:, i].mean() / total:.1f} % |")
    rest = total - rec[:, :len(names)].sum(axis=1).mean()
    print(f"| outside the chunk loop | {rest:.4g} | {100 * rest / total:.1f} % |")
    print(f"| whole kernel | {total:.4g} (min {rec[:, 6].min():.4g}, max {rec[:, 6].max():.4g}) | 100 % |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
