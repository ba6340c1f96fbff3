"""Helpers shared by the GPU parity tests: upload seeded inputs, run the HIP library
through its binding, run the fp64 oracle on the same values, compare."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W

# Acceptance bar: max relative error (fp32 state), per I/O dtype.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def rel_err(y: np.ndarray, r: np.ndarray) -> float:
    """max_i |y_i - r_i| / max(|r_i|, RMS(r)): relative wherever |r_i| >= RMS(r), and measured
    against the output's RMS near zero crossings of sum_n C h + D x."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    if not np.isfinite(y).all():
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), max(rms, 1e-300))
    return float(np.max(np.abs(y - r) / den))


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype: str, device="cuda"):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def f64(a, dtype):
    return None if a is None else W.to_f64(a, dtype)


def run_gpu(kind: str, inp: dict, dtype: str, H=0, Wd=0, softplus=False, use_D=True, use_z=True, use_bias=False,
            stream=None, window=0, zoh=False):
    import selective_state_space_51_amd as S
    x = to_dev(inp["x"], dtype)
    delta = to_dev(inp["w"] if softplus else inp["delta"], dtype)
    A = to_dev(inp["A"], "f32")
    B = to_dev(inp["B"], dtype)
    C = to_dev(inp["C"], dtype)
    D = to_dev(inp["D"], "f32") if use_D else None
    z = to_dev(inp["z"], dtype) if (use_z and inp.get("z") is not None) else None
    bias = to_dev(inp["delta_bias"], "f32") if use_bias else None
    if kind == "selscan":
        y = S.selscan_fwd(x, delta, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=softplus, zoh=zoh,
                          stream=stream)
    elif kind == "bidir":
        y = S.selscan_bidir_fwd(x, delta, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=softplus, zoh=zoh,
                                stream=stream)
    elif kind == "local_ss2d":
        y = S.local_ss2d_fwd(x, delta, A, B, C, H, Wd, window, D=D, z=z, delta_bias=bias, delta_softplus=softplus,
                             zoh=zoh, stream=stream)
    else:
        y = S.ss2d_fwd(x, delta, A, B, C, H, Wd, D=D, z=z, delta_bias=bias, delta_softplus=softplus, zoh=zoh,
                       stream=stream)
    return y


def run_oracle(kind: str, inp: dict, dtype: str, H=0, Wd=0, softplus=False, use_D=True, use_z=True,
               use_bias=False, channels=None, window=0, zoh=False):
    """Oracle on the same values; ``channels`` restricts it to a subset of channels (the scan
    is independent per channel), returning y[..., channels]."""
    sel = slice(None) if channels is None else np.asarray(channels)
    lead = inp["x"].ndim  # 3

    def tok(a):  # per-token arrays [..., dim]
        return None if a is None else f64(a, dtype)[..., sel]

    x = tok(inp["x"])
    delta = tok(inp["w"] if softplus else inp["delta"])
    z = tok(inp.get("z")) if use_z else None
    A = inp["A"].astype(np.float64)[..., sel, :]
    D = inp["D"].astype(np.float64)[..., sel] if use_D else None
    bias = inp["delta_bias"].astype(np.float64)[..., sel] if use_bias else None
    B = f64(inp["B"], dtype)
    C = f64(inp["C"], dtype)
    del lead
    if kind == "selscan":
        return oracle.selscan(x, delta, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=softplus, zoh=zoh)
    if kind == "bidir":
        return oracle.selscan_bidir(x, delta, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=softplus, zoh=zoh)
    if kind == "local_ss2d":
        return oracle.local_ss2d(x, delta, A, B, C, H, Wd, window, D=D, z=z, delta_bias=bias,
                                 delta_softplus=softplus, zoh=zoh)
    return oracle.ss2d(x, delta, A, B, C, H, Wd, D=D, z=z, delta_bias=bias, delta_softplus=softplus, zoh=zoh)
