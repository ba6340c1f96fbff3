#!/usr/bin/env python3
"""Throughput of the selective-scan forward on one MI355X.

A step is one pass of the whole hot path (one selscan_fwd / selscan_bidir_fwd /
ss2d_fwd / local_ss2d_fwd call; with --pass bwd one selscan_scan_bwd call) over one batch
of synthetic input already resident in HBM.
Prints ONE JSON line (rank 0).  Default workload: the Mamba-1.4B-layer
long-context shape, batch 2 x L 65536 x D 4096, N 16, bf16 I/O, fp32 state.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# The headline roofline is HBM: the metric is achieved algorithmic GB/s (every input read once, y
# written once) against the published 8 TB/s.  Beside it, the method's arithmetic per element
# (b, t, d, n, direction): delta*A and (delta*x)*B (2 multiplies), the state update and the output
# term (2 FMAs) = 6 fp32 flops, and one exp2, against the published fp32 vector peak of
# 157.3 TFLOP/s (a figure that counts packed fp32 FMAs, which this build does not emit).
FP32_PEAK_TFLOPS = 157.3
METHOD_FLOPS_PER_ELEMENT = 6
# The backward's method arithmetic per element (the recomputed forward's 6 flops, the adjoint
# g = C*dyp + carry and its decay e*g (4), and the step derivatives e*h_prev, dA, ddelta, dB, dC,
# the dx sum (12)): 22 flops and one exp2.
METHOD_FLOPS_PER_ELEMENT_BWD = 22
# Issue costs on gfx950 in SIMD cycles per wave64 instruction at two waves per SIMD (the scan
# kernels' occupancy), in a stream that mixes v_exp_f32 with FMAs, measured by the committed
# microbenchmark (selective_state_space_51_amd/ubench.py; profiles/ubench_issue_costs_gfx950.md):
# an fp32 FMA/multiply ~4.2, v_exp_f32 ~8.9.  The method floor below is what the method's own 4
# FMA-class operations + 1 exp2 per element take at the measured shader clock on all 1024 SIMDs;
# the two-pass floor adds the one FMA per element this kernel design repeats.
ISSUE_CYCLES_FMA = 4.2
ISSUE_CYCLES_EXP = 8.9
N_SIMDS = 1024
METRIC_BWD = "selective-scan bwd (gradients of x, delta, A, B, C, D, z) B·L·D·N elem/s, 1 GPU"
DEFAULT_WORKLOAD = "mamba1p4b_layer_b2_L65536_D4096"
METRIC = "selective-scan fwd B·L·D·N elem/s + achieved HBM GB/s vs peak, 1 GPU"
LIB_SO = os.path.join(ROOT, "selective_state_space_51_amd", "libselscan.so")
# the kernels (mangled names) a counter record covers, per pass and workload kind; the record is
# valid while their machine code in the built library is unchanged
_FWD = "_ZN12_GLOBAL__N_115selscan_chunkedItLi{k}ELb0ELi{kk}ELi{occ}EEEvNS_6ParamsE"
_BWD = ("_ZN12_GLOBAL__N_119selscan_bwd_chunkedItLi{k}ELb0EEEvNS_9BwdParamsE",
        "_ZN12_GLOBAL__N_118selscan_bwd_reduceItLi{k}EEEvNS_15BwdReduceParamsE")
_KIND = {"selscan": 0, "bidir": 1, "ss2d": 2, "local_ss2d": 3}


_MERGE = "_ZN12_GLOBAL__N_113selscan_mergeItEEvNS_11MergeParamsE"


def fwd_occ3(kind: str, seqlen: int, batch: int, dim: int, cus: int, split: bool = False) -> bool:
    """Whether the library launches its three-workgroup forward (the rule in selscan_fwd.hip,
    Euler Bbar, bf16 io): more than 208 steps, and 1.25 r3 < r2 for the rounds of workgroups at
    three (r3) and two (r2) per compute unit (a direction-split grid has a workgroup per direction
    and tile)."""
    g = batch * (-(-dim // 16)) * ({"selscan": 1, "bidir": 2}.get(kind, 4) if split else 1)
    r2, r3 = -(-g // (2 * cus)), -(-g // (3 * cus))
    return seqlen > 208 and 5 * r3 < 4 * r2


def profiled_kernels(pass_: str, kind: str, seqlen: int = 1 << 30, split: bool = False, occ3: bool = False):
    k = _KIND[kind]
    if pass_ == "fwd":
        # sequences of at most 208 steps run the 13-steps-per-lane instance; a direction-split
        # grid adds the merge of the directions' rows
        kk = 13 if seqlen <= 208 else 16
        return [_FWD.format(k=k, kk=kk, occ=3 if occ3 and kk == 16 else 2)] + ([_MERGE] if split else [])
    if pass_ == "bwd":
        return [n.format(k=k) for n in _BWD]
    if kind in ("ss2d", "local_ss2d"):
        return ["_ZN12_GLOBAL__N_116dwconv2d3_kernelItEEvNS_10Dw2dParamsE"]
    return ["_ZN12_GLOBAL__N_120causal_conv1d_kernelItLi4EEEvNS_12Conv1dParamsE"]


def kernel_code_hash(names, so_path: str = LIB_SO) -> str:
    """sha256[:16] over the gfx950 machine code and kernel descriptors of the named kernels, read
    from the code objects embedded in the built library (clang offload bundles; ELF symbol table).
    The descriptors' code-entry offsets are left out: they change when other kernels of the same
    code object move the code, not when the kernel's own code changes."""
    import struct
    data = open(so_path, "rb").read()
    want = set(names) | {n + ".kd" for n in names}
    found = {}
    i = data.find(b"__CLANG_OFFLOAD_BUNDLE__")
    while i >= 0:
        n = struct.unpack_from("<Q", data, i + 24)[0]
        off = i + 32
        for _ in range(n):
            eo, esz, tl = struct.unpack_from("<QQQ", data, off)
            triple = data[off + 24:off + 24 + tl]
            off += 24 + tl
            if b"gfx950" not in triple or esz == 0:
                continue
            elf = data[i + eo:i + eo + esz]
            shoff, = struct.unpack_from("<Q", elf, 0x28)
            shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
            secs = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + j * shentsize) for j in range(shnum)]
            for sec in secs:
                if sec[1] != 2:  # SHT_SYMTAB
                    continue
                strtab = secs[sec[6]]
                for j in range(sec[5] // 24):
                    st_name, st_info, st_other, st_shndx, st_value, st_size = struct.unpack_from(
                        "<IBBHQQ", elf, sec[4] + j * 24)
                    end = elf.index(b"\0", strtab[4] + st_name)
                    name = elf[strtab[4] + st_name:end].decode()
                    if name in want and st_shndx < shnum and st_size:
                        home = secs[st_shndx]
                        start = home[4] + (st_value - home[3])  # file offset = sh_offset + (vaddr - sh_addr)
                        body = elf[start:start + st_size]
                        if name.endswith(".kd") and len(body) >= 24:
                            # the descriptor's code-entry offset (bytes 16..23) moves with the
                            # layout of the code object, not with the kernel's own code
                            body = body[:16] + bytes(8) + body[24:]
                        found[name] = body
        i = data.find(b"__CLANG_OFFLOAD_BUNDLE__", i + 1)
    if set(found) != want:
        return "missing:" + ",".join(sorted(want - set(found)))[:60]
    h = hashlib.sha256()
    for name in sorted(found):
        h.update(name.encode())
        h.update(found[name])
    return h.hexdigest()[:16]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_clock_prepare(S, torch, op, w, dev, launches: int):
    """Stamp buffers and events for `kernel_clock`, allocated before the timed region so that the
    clocked launches follow its last launch without an idle gap (after a few milliseconds of idle
    the shader clock drops and takes about ten launches to climb back)."""
    nb = S.selscan_clock_stamps_bytes(op, w.batch, w.dim)
    bufs = [torch.zeros(nb // 8, dtype=torch.int64, device=dev) for _ in range(launches)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    return bufs, ev


def kernel_clock(torch, run, prepared):
    """Shader clock of the scan kernel itself: back-to-back calls of the clocked forward (the timed
    code path plus two counter reads and four stores per workgroup), enqueued right after the timed
    region's closing synchronize; per workgroup the s_memtime (shader clock) and s_memrealtime
    (100 MHz) counters at its start and end.  Returns the clock in MHz weighted by workgroup time,
    with the kernel time of those launches."""
    bufs, ev = prepared
    stream = torch.cuda.current_stream()
    for (a, b), s in zip(ev, bufs):
        a.record(stream)
        run(s)
        b.record(stream)
    torch.cuda.synchronize()
    clk = rt = 0.0
    for s in bufs:
        v = s.view(-1, 4).double()
        used = v[:, 3] > 0  # workgroups of the grid (a direction-split grid fills every slot)
        clk += float((v[used, 1] - v[used, 0]).sum())
        rt += float((v[used, 3] - v[used, 2]).sum())
    ms = [a.elapsed_time(b) for a, b in ev]
    return {"sclk_mhz": clk / (rt / 1e8) / 1e6 if rt > 0 else None, "launches": len(bufs),
            "kernel_ms": sum(ms) / len(ms),
            "source": "in-kernel s_memtime / s_memrealtime of selscan_chunked (selscan_scan_fwd_clocked), "
                      "launched right after the timed region"}


def memory_clock_mhz():
    """The HBM clock the driver reports as current (the level marked '*' in the card's
    pp_dpm_mclk), read once after the timed region; None where the file is not readable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_mclk")):
        try:
            for line in open(path):
                if "*" in line:
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            continue
    return None


def bwd_algorithmic_bytes(w) -> int:
    """Bytes a fused backward must move at least once: x, dy, z and each direction's delta and
    chunk states read, dx, dz and each direction's ddelta written (io dtype); each direction's
    B, C read and dB, dC written; A, D read and dA, dD written per direction."""
    s, k = w.io_bytes, w.ndir
    tok = w.batch * w.seqlen * w.dim
    bc = w.batch * w.seqlen * w.dstate * s
    ck = k * w.batch * ((w.seqlen + 255) // 256) * w.dim * w.dstate * 4
    params = 2 * k * (w.dim * w.dstate + w.dim) * 4
    g = 1 if w.gate else 0
    return tok * s * ((2 + k + g) + (1 + k + g)) + 4 * k * bc + ck + params


def measured_traffic(workload: str, pass_: str = "fwd", kind: str = "selscan", seqlen: int = 1 << 30,
                     split: bool = False, occ3: bool = False):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    kernels' current machine code; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(workload + ("" if pass_ == "fwd" else "/" + pass_))
    if not e or e.get("kernel_code_sha") != kernel_code_hash(profiled_kernels(pass_, kind, seqlen, split, occ3)):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, budget_channels: int, threads: int = 0):
    """The fp64 oracle as it stands, on all host cores (or `threads`), on a bounded sample of the
    workload: every batch row and the whole sequence for the first `budget_channels` channels."""
    import numpy as np

    import oracle
    import workloads as W

    inp = W.generate(w)
    ch = min(budget_channels, w.dim)
    f = lambda k: None if inp.get(k) is None else np.ascontiguousarray(W.to_f64(inp[k], w.dtype)[..., :ch])
    x, dl, z = f("x"), f("delta"), f("z")
    A = inp["A"].astype(np.float64)[..., :ch, :]
    D = inp["D"].astype(np.float64)[..., :ch]
    B, C = W.to_f64(inp["B"], w.dtype), W.to_f64(inp["C"], w.dtype)
    del inp
    threads = threads or oracle.default_threads()
    t0 = time.perf_counter()
    if w.kind == "selscan":
        oracle.selscan(x, dl, A, B, C, D=D, z=z, nthreads=threads)
    elif w.kind == "bidir":
        oracle.selscan_bidir(x, dl, A, B, C, D=D, z=z, nthreads=threads)
    elif w.kind == "local_ss2d":
        oracle.local_ss2d(x, dl, A, B, C, w.H, w.W, w.window, D=D, z=z, nthreads=threads)
    else:
        oracle.ss2d(x, dl, A, B, C, w.H, w.W, D=D, z=z, nthreads=threads)
    sec = time.perf_counter() - t0
    elems = w.batch * w.seqlen * ch * w.dstate * w.ndir
    return {
        "value": elems / sec,
        "unit": "elem/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{w.name}: all {w.batch} batch rows x {w.seqlen} steps x first {ch} of {w.dim} channels"
                  f" x {w.ndir} direction(s) ({elems:.3e} elements, {sec:.1f} s wall, fp64)",
    }


def cpu_baseline_bwd(w, budget_channels: int):
    """The fp64 oracle backward (all host cores) on a bounded sample: every batch row and the whole
    sequence for the first `budget_channels` channels (dB, dC then sum over those channels only;
    the work per element is the same)."""
    import numpy as np

    import oracle
    import workloads as W

    inp = W.generate(w)
    ch = min(budget_channels, w.dim)
    f = lambda a: None if a is None else np.ascontiguousarray(W.to_f64(a, w.dtype)[..., :ch])
    x, dl, z = f(inp["x"]), f(inp["delta"]), f(inp.get("z"))
    dy = f(W.generate_cotangent(w.batch, w.seqlen, w.dim, w.dtype))
    A = np.ascontiguousarray(inp["A"].astype(np.float64)[..., :ch, :])
    D = np.ascontiguousarray(inp["D"].astype(np.float64)[..., :ch])
    B, C = W.to_f64(inp["B"], w.dtype), W.to_f64(inp["C"], w.dtype)
    del inp
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    if w.kind == "selscan":
        oracle.selscan_bwd(x, dl, A, B, C, dy, D=D, z=z, nthreads=threads)
    else:
        oracle.multi_bwd(w.kind, x, dl, A, B, C, dy, D=D, z=z, H=w.H, W=w.W, window=w.window, nthreads=threads)
    sec = time.perf_counter() - t0
    elems = w.batch * w.seqlen * ch * w.dstate * w.ndir
    return {"value": elems / sec, "unit": "elem/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{w.name} backward: all {w.batch} batch rows x {w.seqlen} steps x first {ch} of {w.dim} "
                      f"channels x {w.ndir} direction(s) ({elems:.3e} elements, {sec:.1f} s wall, fp64)"}


def cpu_baseline_conv(w, g, two_d: bool, budget_channels: int):
    """The fp64 oracle convolution (one host thread: the oracle's direct sum is not threaded) on
    every batch row and position of the first `budget_channels` channels."""
    import numpy as np

    import oracle
    import workloads as W

    ch = min(budget_channels, w.dim)
    x = np.ascontiguousarray(W.to_f64(g["x"], w.dtype)[..., :ch])
    wt = np.ascontiguousarray(g["weight"][:ch].astype(np.float64))
    bias = g["bias"][:ch].astype(np.float64)
    t0 = time.perf_counter()
    if two_d:
        oracle.dwconv2d(x, wt, w.H, w.W, bias=bias, silu=True)
    else:
        oracle.causal_conv1d(x, wt, bias=bias, silu=True)
    sec = time.perf_counter() - t0
    elems = w.batch * w.seqlen * ch
    return {"value": elems / sec, "unit": "elem/s", "cores": 1, "kind": "oracle",
            "sample": f"{w.name} {'3x3' if two_d else 'k=4'} convolution: all {w.batch} batch rows x {w.seqlen} "
                      f"positions x first {ch} of {w.dim} channels ({elems:.3e} elements, {sec:.1f} s wall, fp64)"}


METRIC_CONV = "conv prologue (depthwise conv + SiLU) B·L·D elem/s + achieved HBM GB/s vs peak, 1 GPU"
METRIC_CONV_BWD = "conv prologue backward (dx, dweight, dbias) B·L·D elem/s + achieved HBM GB/s vs peak, 1 GPU"


def conv_bench(args, w, S, W, torch, np, up, dev) -> int:
    """--pass conv: the depthwise convolution + SiLU in front of the scan, on the workload's x shape
    (k = 4 causal along the sequence for 1-D workloads; 3x3 on the H x W map for 2-D ones);
    --pass conv_bwd: its backward (dx, dweight, dbias from dout)."""
    two_d = w.kind in ("ss2d", "local_ss2d")
    width = 3 if two_d else 4
    bwd = args.pass_ == "conv_bwd"
    g = W.generate_conv(w.batch, w.seqlen, w.dim, width, w.dtype, two_d=two_d)
    x, wt, bias = up(g["x"]), up(g["weight"]), up(g["bias"])
    out = up(W.generate_cotangent(w.batch, w.seqlen, w.dim, w.dtype)) if bwd else torch.empty_like(x)
    stream = torch.cuda.current_stream()
    # rotate over copies of x and out (dout for the backward) totalling at least 512 MiB when one
    # pair would fit in the 256 MB Infinity Cache (as the scan passes do)
    pair = 2 * x.numel() * x.element_size()
    copies = 1 if args.no_rotate or pair >= (512 << 20) else min(64, -(-(512 << 20) // pair))
    xs = [(x, out)] + [(x.clone(), out.clone() if bwd else torch.empty_like(out)) for _ in range(copies - 1)]
    if bwd:
        code = S.SELSCAN_BF16 if w.dtype == "bf16" else S.SELSCAN_F32
        need = (S.dwconv2d_bwd_workspace_bytes(w.batch, w.H, w.W, w.dim, code) if two_d else
                S.causal_conv1d_bwd_workspace_bytes(w.batch, w.seqlen, w.dim, width, code))
        cws = torch.empty(need, dtype=torch.uint8, device=dev)
    if bwd and two_d:
        step = lambda i: S.dwconv2d_bwd(xs[i % copies][0], wt, w.H, w.W, xs[i % copies][1], bias=bias, workspace=cws,
                                        stream=stream)
    elif bwd:
        step = lambda i: S.causal_conv1d_bwd(xs[i % copies][0], wt, xs[i % copies][1], bias=bias, workspace=cws,
                                             stream=stream)
    elif two_d:
        step = lambda i: S.dwconv2d_fwd(xs[i % copies][0], wt, w.H, w.W, bias=bias, out=xs[i % copies][1],
                                        stream=stream)
    else:
        step = lambda i: S.causal_conv1d_fwd(xs[i % copies][0], wt, bias=bias, out=xs[i % copies][1], stream=stream)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(args.warmup + i)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    kern_ms = float(np.mean(launch_ms))
    ms_step = wall * 1e3 / args.steps
    elems = w.batch * w.seqlen * w.dim
    taps = width * (width if two_d else 1)
    # algorithmic bytes: x read once, out written once, the filters and biases read once; the
    # backward reads x and dout, writes dx, reads the filters and writes their gradients
    alg = (3 if bwd else 2) * elems * w.io_bytes + w.dim * (taps + 1) * 4 * (2 if bwd else 1)
    gbs = alg / (kern_ms * 1e-3) / 1e9
    if bwd:
        kname = ("dwconv2d3_bwd_dv + dwconv2d3_bwd_dx + conv_bwd_reduce" if two_d else
                 "conv1d_bwd_dv + conv1d_bwd_dx + conv_bwd_reduce")
    else:
        kname = "dwconv2d3_kernel" if two_d else "causal_conv1d_kernel"
    out_line = {
        "metric": METRIC_CONV_BWD if bwd else METRIC_CONV, "value": elems / (ms_step * 1e-3), "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded: x ~ N(0,1); filter ~ N(0, 1/taps); bias ~ N(0,1))",
        "config": {"workload": w.name, "kind": "dwconv2d_3x3" if two_d else "causal_conv1d_k4", "batch": w.batch,
                   "seqlen": w.seqlen, "dim": w.dim, "io_dtype": w.dtype, "silu": True, "pass": args.pass_,
                   "input_sets": copies},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None if bwd else measured_traffic(w.name, "conv", w.kind), "kernel": kname,
                     "kernel_ms": kern_ms,
                     "kernel_ms_min": float(np.min(launch_ms)), "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline and not bwd:
        del x, out, xs
        torch.cuda.empty_cache()
        out_line["cpu_baseline"] = cpu_baseline_conv(w, g, two_d, min(args.cpu_channels, 1024))
    print(json.dumps(out_line))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the shader clock ramps up over the first ~10 launches after an idle moment (up to 15 %
    # slower at first): the default warm-up covers it
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd", "conv", "conv_bwd"], default="fwd",
                    help="fwd: the forward scan (default); bwd: selscan_scan_bwd (gradients of every input, "
                         "states recomputed from the chunk states a forward saved beforehand); conv: the "
                         "convolution in front of the scan (causal conv1d k=4 + SiLU for the 1-D workloads, "
                         "DWConv 3x3 + SiLU for the 2-D ones) on the workload's x; conv_bwd: its backward")
    ap.add_argument("--state", action="store_true",
                    help="single-direction workloads: run selscan_fwd_state with an initial state and the "
                         "final state written (recurrent / chunked inference)")
    ap.add_argument("--zoh", action="store_true",
                    help="forward with the zero-order-hold Bbar (SELSCAN_FLAG_ZOH) instead of delta * B")
    ap.add_argument("--softplus", action="store_true",
                    help="pass the pre-activation w and a per-channel bias with delta_softplus=1, so the "
                         "kernels form delta = softplus(w + bias) themselves (w drawn so that delta has the "
                         "workload's distribution); no CPU baseline is taken with it")
    ap.add_argument("--no-rotate", action="store_true",
                    help="time every step on the same input and output buffers, even when they would fit in "
                         "the 256 MB Infinity Cache (by default such workloads rotate over copies totalling "
                         "at least 512 MiB)")
    ap.add_argument("--cpu-channels", type=int, default=4096)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the CPU baseline (default: all cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one device copy of 1 GiB (a plain copy of known size, for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the scan shards over batch x channel with no "
              f"communication); --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import selective_state_space_51_amd as S
    import workloads as W

    w = W.by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.generate(w, with_w=args.softplus, with_bias=args.softplus)
    if args.softplus:
        inp["delta"] = inp.pop("w")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    t = {k: up(v) for k, v in inp.items()}
    del inp
    y = torch.empty_like(t["x"])
    ws = None
    op = {"selscan": S.SELSCAN_OP_FWD, "bidir": S.SELSCAN_OP_BIDIR, "ss2d": S.SELSCAN_OP_SS2D,
          "local_ss2d": S.SELSCAN_OP_LOCAL_SS2D}[w.kind]
    need = S.selscan_workspace_bytes(op, w.batch, w.seqlen, w.dim, w.dstate,
                                     S.SELSCAN_BF16 if w.dtype == "bf16" else S.SELSCAN_F32)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.zoh and args.pass_ in ("conv", "conv_bwd"):
        print("--zoh applies to the scan passes only", file=sys.stderr)
        return 2
    if args.pass_ in ("conv", "conv_bwd"):
        return conv_bench(args, w, S, W, torch, np, up, dev)
    if args.state and w.kind != "selscan":
        print("--state applies to single-direction workloads only", file=sys.stderr)
        return 2
    h0 = hl = None
    if args.state:
        h0 = up(W.generate_state(w.batch, w.dim, w.dstate))
        hl = torch.empty_like(h0)

    bws = None
    geo = dict(H=w.H, W=w.W, window=w.window)
    bwd = args.pass_ == "bwd"
    # Input sets: the workload's tensors, and for workloads whose buffers would fit in the 256 MB
    # Infinity Cache, copies of them (with their own outputs) up to 512 MiB in all (at most 64
    # sets), which the steps rotate over so that every step streams its inputs from HBM.
    first = dict(t=t, y=y)
    if bwd:
        _, first["ck"] = S.selscan_scan_fwd(op, t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                            y=y, chunk_states=True, workspace=ws, stream=stream, **geo,
                                            delta_bias=t.get("delta_bias"), delta_softplus=args.softplus,
                                            zoh=args.zoh)
        first["dy"] = up(W.generate_cotangent(w.batch, w.seqlen, w.dim, w.dtype))
        bws = torch.empty(S.selscan_scan_bwd_workspace_bytes(op, w.batch, w.seqlen, w.dim, w.dstate,
                                                             S.SELSCAN_BF16 if w.dtype == "bf16" else S.SELSCAN_F32),
                          dtype=torch.uint8, device=dev)
    run_bwd = lambda c, g=None: S.selscan_scan_bwd(
        op, c["t"]["x"], c["t"]["delta"], c["t"]["A"], c["t"]["B"], c["t"]["C"], c["dy"], c["ck"], D=c["t"]["D"],
        z=c["t"]["z"], workspace=bws, stream=stream, delta_bias=c["t"].get("delta_bias"),
        delta_softplus=args.softplus, zoh=args.zoh, grads=g, **geo)
    nbytes = lambda d: sum(v.numel() * v.element_size() for v in d.values() if isinstance(v, torch.Tensor))
    set_bytes = nbytes(t) + y.numel() * y.element_size()
    if bwd:
        first["g"] = run_bwd(first)  # the gradient buffers of the first set
        set_bytes += nbytes({"ck": first["ck"], "dy": first["dy"]}) + nbytes(first["g"])
    rotate_to = 512 << 20
    copies = 1 if args.no_rotate or set_bytes >= rotate_to else min(64, -(-rotate_to // set_bytes))
    sets = [first]
    for _ in range(copies - 1):
        c = dict(t={k: None if v is None else v.clone() for k, v in t.items()}, y=torch.empty_like(y))
        if bwd:
            c["ck"], c["dy"] = first["ck"].clone(), first["dy"].clone()
            c["g"] = run_bwd(c)  # each set writes its own gradient buffers
        sets.append(c)
    torch.cuda.synchronize()

    def step(i):
        c = sets[i % copies]
        t, y = c["t"], c["y"]
        dkw = dict(delta_bias=t.get("delta_bias"), delta_softplus=args.softplus)
        if bwd:
            run_bwd(c, c["g"])
        elif args.state:
            S.selscan_fwd_state(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], y=y, h0=h0,
                                h_last=hl, workspace=ws, zoh=args.zoh, stream=stream, **dkw)
        elif w.kind == "selscan":
            S.selscan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], y=y, workspace=ws,
                          zoh=args.zoh, stream=stream, **dkw)
        elif w.kind == "bidir":
            S.selscan_bidir_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], y=y,
                                workspace=ws, zoh=args.zoh, stream=stream, **dkw)
        elif w.kind == "local_ss2d":
            S.local_ss2d_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], w.H, w.W, w.window, D=t["D"], z=t["z"], y=y,
                             workspace=ws, zoh=args.zoh, stream=stream, **dkw)
        else:
            S.ss2d_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], w.H, w.W, D=t["D"], z=t["z"], y=y,
                       workspace=ws, zoh=args.zoh, stream=stream, **dkw)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    clocked = not bwd and not args.state
    prepared = kernel_clock_prepare(S, torch, op, w, dev, min(args.steps, 10)) if clocked else None
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch events on the stream the kernel runs on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(args.warmup + i)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the shader clock of the same kernel, over launches right after the timed region
    clock = None
    if clocked:
        c0 = sets[0]["t"]
        clock = kernel_clock(torch, lambda s: S.selscan_scan_fwd_clocked(
            op, c0["x"], c0["delta"], c0["A"], c0["B"], c0["C"], s, D=c0["D"], z=c0["z"], y=sets[0]["y"],
            workspace=ws, zoh=args.zoh, delta_bias=c0.get("delta_bias"), delta_softplus=args.softplus, stream=stream,
            **geo), prepared)
        clock["mclk_mhz"] = memory_clock_mhz()
        clock["mclk_source"] = "current level of the card's pp_dpm_mclk (sysfs), after the timed region"
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean(launch_ms))
    value = w.elements / (ms_step * 1e-3)
    alg = bwd_algorithmic_bytes(w) if bwd else w.algorithmic_bytes()
    if args.softplus:
        alg += (2 if bwd else 1) * w.ndir * w.dim * 4  # the delta bias read (and its gradient written)
    hbm_gbs = alg / (kern_ms * 1e-3) / 1e9
    flops = w.elements * (METHOD_FLOPS_PER_ELEMENT_BWD if bwd else METHOD_FLOPS_PER_ELEMENT)
    tflops = flops / (kern_ms * 1e-3) / 1e12
    # the method's own issue floor: 4 VALU operations and 1 exp2 per element on every SIMD at the
    # measured shader clock (forward, Euler Bbar); this kernel design adds one FMA per element
    # (its second pass over a lane's steps) to that
    sclk = clock.get("sclk_mhz") if clock else None
    floor = None
    if sclk and not bwd and not args.zoh:
        cyc = w.elements / (64 * N_SIMDS) * (4 * ISSUE_CYCLES_FMA + ISSUE_CYCLES_EXP)
        cyc2 = w.elements / (64 * N_SIMDS) * (5 * ISSUE_CYCLES_FMA + ISSUE_CYCLES_EXP)
        floor = {"method_ms": cyc / (sclk * 1e3), "two_pass_ms": cyc2 / (sclk * 1e3),
                 "cycles_per_element": {"fma": ISSUE_CYCLES_FMA, "exp": ISSUE_CYCLES_EXP},
                 "simds": N_SIMDS, "sclk_mhz": sclk}
    # the counter record is for the plain call of the pass (no state in/out, Euler Bbar, delta as given)
    split = w.ndir > 1 and w.batch * (-(-w.dim // 16)) < 1024
    occ3 = not bwd and w.dtype == "bf16" and fwd_occ3(
        w.kind, w.seqlen, w.batch, w.dim, torch.cuda.get_device_properties(0).multi_processor_count, split)
    traffic = None if (args.zoh or args.state or args.softplus) else measured_traffic(
        w.name, args.pass_, w.kind, w.seqlen, split and args.pass_ == "fwd", occ3)
    if bwd:
        kname = "selscan_bwd_chunked + selscan_bwd_merge + selscan_bwd_reduce" if split else \
            "selscan_bwd_chunked + selscan_bwd_reduce"
    else:
        kname = "selscan_chunked + selscan_merge" if split else "selscan_chunked"
    out = {
        "metric": METRIC_BWD if bwd else METRIC,
        "value": value,
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: x, z, B, C ~ N(0,1); delta log-uniform [1e-3, 1e-1]; A[d,n] = -(n+1); D ~ N(0,1))",
        "config": {"workload": w.name, "kind": w.kind, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "directions": w.ndir, "io_dtype": w.dtype, "gate": w.gate,
                   "window": w.window or None,
                   "state_io": bool(args.state), "pass": args.pass_, "bbar": "zoh" if args.zoh else "delta*B",
                   "delta_softplus": bool(args.softplus), "input_sets": copies},
        "roofline": {"bound": "hbm", "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hbm_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "kernel_ms": kern_ms, "kernel_ms_median": float(np.median(launch_ms)),
                     "kernel_ms_min": float(np.min(launch_ms)),
                     "elements_per_launch": w.elements, "algorithmic_bytes_per_launch": alg,
                     "flops_per_element": METHOD_FLOPS_PER_ELEMENT_BWD if bwd else METHOD_FLOPS_PER_ELEMENT,
                     "flop_achieved_TFLOPs": tflops, "flop_peak_TFLOPs": FP32_PEAK_TFLOPS,
                     "flop_frac": tflops / FP32_PEAK_TFLOPS, "issue_floor": floor},
        "clock": clock,
    }
    if not args.no_cpu_baseline and not args.softplus and bwd:
        del t, y, ws, h0, hl, first, sets, bws
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline_bwd(w, min(args.cpu_channels, 2048))
    elif not args.no_cpu_baseline and not args.softplus:
        del t, y, ws, h0, hl, first, sets
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_channels, args.cpu_threads)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
