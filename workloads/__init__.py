"""Seeded synthetic inputs for the selective-scan workloads.

This module holds no arithmetic of the method: it only draws random
numbers, rounds them to the I/O dtype and names the workload shapes.  It is
the one piece shared by the CPU oracle side (tests, CPU baseline) and the
HIP side (tests, bench), so both always see bit-identical inputs.

Value distributions (plainest reading of the workload statements; the
pages print no activation statistics):
  x, z, B, C ~ N(0, 1)             activations, drawn in float32
  D[d]       ~ N(0, 1)             per-channel skip weight (float32)
  A[d, n]    = -(n + 1)            real, negative, diagonal (S4D-real style)
  delta      = exp(U(ln 1e-3, ln 1e-1))   log-uniform step size
  w          = log(expm1(delta))   pre-softplus value (softplus(w) == delta)
Every direction of the bidirectional / SS2D workloads draws its own delta,
B and C.  The 16-bit ``bf16`` arrays are raw IEEE bfloat16 bit patterns
(round-to-nearest-even from float32), held as numpy uint16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

SEED_BASE = 51000


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload shape.  ``kind`` is 'selscan', 'bidir' or 'ss2d'."""

    name: str
    kind: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str  # 'f32' or 'bf16' (I/O dtype of x, delta, B, C, z, y)
    gate: bool  # whether z is passed
    H: int = 0
    W: int = 0
    index: int = 0  # position in WORKLOADS; the seed is SEED_BASE + index
    window: int = 0  # window side of the windowed cross-scan

    @property
    def ndir(self) -> int:
        return {"selscan": 1, "bidir": 2, "ss2d": 4, "local_ss2d": 4}[self.kind]

    @property
    def elements(self) -> int:
        """batch * L * D * N * directions: the unit the throughput metric counts."""
        return self.batch * self.seqlen * self.dim * self.dstate * self.ndir

    @property
    def io_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self) -> int:
        """Bytes a fused forward must move at least once: every input read once, y written once.

        x once, delta once per direction, z once (if gated), y once, B and C once per
        direction, A (D*N fp32) and D (fp32) once per direction.
        """
        s = self.io_bytes
        tok = self.batch * self.seqlen * self.dim
        k = self.ndir
        big = tok * s * (1 + k + (1 if self.gate else 0) + 1)
        bc = k * 2 * self.batch * self.seqlen * self.dstate * s
        params = k * (self.dim * self.dstate + self.dim) * 4
        return big + bc + params


WORKLOADS: List[Workload] = [
    Workload("s6_fp32_b1_L256_D16", "selscan", 1, 256, 16, 16, "f32", True, index=0),
    Workload("mamba130m_layer_b8_L2048_D1536", "selscan", 8, 2048, 1536, 16, "bf16", True, index=1),
    Workload("mamba1p4b_layer_b2_L65536_D4096", "selscan", 2, 65536, 4096, 16, "bf16", True, index=2),
    Workload("vim_bidir_b64_L197_D768", "bidir", 64, 197, 768, 16, "bf16", True, index=3),
    Workload("vmamba_ss2d_b32_56x56_D192", "ss2d", 32, 56 * 56, 192, 16, "bf16", False, H=56, W=56, index=4),
    # the windowed cross-scan on the VMamba stage-1 map, windows of 7 x 7 pixels
    Workload("localmamba_local_ss2d_b32_56x56_w7_D192", "local_ss2d", 32, 56 * 56, 192, 16, "bf16", False, H=56, W=56,
             index=5, window=7),
    # a video clip of 8 frames of 14 x 14 patches scanned spatial-first in both directions (the
    # bidirectional scan on the frame-major token sequence), at an inner width of 768 channels
    Workload("videomamba_bidir_b16_T8x14x14_D768", "bidir", 16, 8 * 14 * 14, 768, 16, "bf16", True, index=6),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (NaN kept quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of an I/O array (bf16 bits or float32) to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


_BLOCK = 1 << 22  # elements per independently seeded block


def _round_io(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _rne_bits(a: np.ndarray, out: np.ndarray) -> None:
    """float32 block (finite by construction) -> bf16 bits, round to nearest even, into out."""
    u = a.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out[:] = r


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


_POOL = None


def _draw_io(seed: int, tensor_id: int, shape, dtype: str, draw) -> np.ndarray:
    """Fill a tensor block by block.  Block j of tensor ``tensor_id`` draws from its own PCG64
    stream seeded by SeedSequence([seed, tensor_id, j]), so the values do not depend on how
    many threads fill the blocks."""
    size = int(np.prod(shape))
    out = np.empty(size, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(j):
        s = j * _BLOCK
        e = min(size, s + _BLOCK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, j])))
        a = draw(rng, e - s)
        if dtype == "bf16":
            _rne_bits(a, out[s:e])
        else:
            out[s:e] = a

    nblk = (size + _BLOCK - 1) // _BLOCK
    if nblk <= 1:
        for j in range(nblk):
            fill(j)
    else:
        list(_pool().map(fill, range(nblk)))
    return out.reshape(shape)


def _std_normal(rng, n):
    return rng.standard_normal(n, dtype=np.float32)


def _normal(seed, tensor_id, shape, dtype: str = "f32") -> np.ndarray:
    return _draw_io(seed, tensor_id, shape, dtype, _std_normal)


def _log_uniform(seed, tensor_id, shape, lo: float, hi: float, dtype: str = "f32") -> np.ndarray:
    a, b = np.float32(math.log(lo)), np.float32(math.log(hi) - math.log(lo))

    def draw(rng, n):
        u = rng.random(n, dtype=np.float32)
        u *= b
        u += a
        return np.exp(u, out=u)

    return _draw_io(seed, tensor_id, shape, dtype, draw)


def generate(
    w: Workload,
    seed: Optional[int] = None,
    with_w: bool = False,
    with_bias: bool = False,
    batch: Optional[int] = None,
    seqlen: Optional[int] = None,
    dim: Optional[int] = None,
) -> Dict[str, np.ndarray]:
    """Draw one seeded input set for workload ``w`` (shape overrides allowed for small cases).

    Returns a dict with keys x, z (or None), delta, A, B, C, D and optionally
    w (pre-softplus delta, for delta_softplus=1 runs) and delta_bias.  Per-
    direction arrays carry a leading direction axis when ``w.ndir > 1``;
    per-token/per-pixel arrays are in token (pixel, row-major) order.
    """
    seed = SEED_BASE + w.index if seed is None else seed
    bt = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    d = w.dim if dim is None else dim
    n = w.dstate
    k = w.ndir
    lead = (k,) if k > 1 else ()
    out: Dict[str, np.ndarray] = {}
    out["x"] = _normal(seed, 0, (bt, L, d), w.dtype)
    out["z"] = _normal(seed, 1, (bt, L, d), w.dtype) if w.gate else None
    out["delta"] = _log_uniform(seed, 2, lead + (bt, L, d), 1e-3, 1e-1, w.dtype)
    out["B"] = _normal(seed, 3, lead + (bt, L, n), w.dtype)
    out["C"] = _normal(seed, 4, lead + (bt, L, n), w.dtype)
    out["D"] = _normal(seed, 5, lead + (d,))
    A = -np.arange(1, n + 1, dtype=np.float32)
    out["A"] = np.ascontiguousarray(np.broadcast_to(A, lead + (d, n)))
    if with_bias:
        out["delta_bias"] = (np.float32(0.5) * _normal(seed, 6, lead + (d,))).astype(np.float32)
    if with_w:
        # pre-softplus value such that softplus(w + bias) ~= delta; computed in fp64 from the
        # delta actually stored, then rounded to the I/O dtype.
        dl = to_f64(out["delta"], w.dtype)
        wv = np.log(np.expm1(dl))
        if with_bias:
            wv = wv - out["delta_bias"].astype(np.float64).reshape(lead + (1, 1, d))
        out["w"] = _round_io(wv.astype(np.float32), w.dtype)
    return out


def generate_periodic(seqlen: int, dim: int, period: int, dtype: str = "bf16", dstate: int = 16, ndir: int = 1,
                      batch: int = 1, seed: int = SEED_BASE + 70) -> Dict[str, np.ndarray]:
    """Inputs too large to draw whole: the per-token tensors x, z, delta and a cotangent dy are
    given as seeded blocks of ``period`` values, element i of the full tensor (row-major; delta
    [ndir, batch, seqlen, dim] with ndir > 1, else [batch, seqlen, dim]) being element i mod
    period of its block; B and C ([ndir,] batch, seqlen, dstate), A and D are drawn whole, with
    the distributions of ``generate``."""
    lead = (ndir,) if ndir > 1 else ()
    out: Dict[str, np.ndarray] = {}
    out["x"] = _normal(seed, 0, (period,), dtype)
    out["z"] = _normal(seed, 1, (period,), dtype)
    out["delta"] = _log_uniform(seed, 2, (period,), 1e-3, 1e-1, dtype)
    out["dy"] = _normal(seed, 7, (period,), dtype)
    out["B"] = _normal(seed, 3, lead + (batch, seqlen, dstate), dtype)
    out["C"] = _normal(seed, 4, lead + (batch, seqlen, dstate), dtype)
    out["D"] = _normal(seed, 5, lead + (dim,))
    A = -np.arange(1, dstate + 1, dtype=np.float32)
    out["A"] = np.ascontiguousarray(np.broadcast_to(A, lead + (dim, dstate)))
    return out


def generate_state(batch: int, dim: int, dstate: int = 16, seed: int = SEED_BASE + 50) -> np.ndarray:
    """A seeded initial state h0 ~ N(0, 1), fp32 [batch][dim][dstate] (for the state-in/out
    entry point)."""
    return _normal(seed, 7, (batch, dim, dstate))


def generate_cotangent(batch: int, seqlen: int, dim: int, dtype: str, seed: int = SEED_BASE + 60) -> np.ndarray:
    """A seeded upstream gradient dL/dy ~ N(0, 1) of the output's shape and I/O dtype (for the
    backward pass)."""
    return _normal(seed, 8, (batch, seqlen, dim), dtype)


def generate_conv(batch: int, seqlen: int, dim: int, width: int, dtype: str, two_d: bool = False,
                  seed: int = SEED_BASE + 70) -> Dict[str, np.ndarray]:
    """Seeded inputs of the convolution in front of the scan: x ~ N(0, 1) [batch, seqlen, dim]
    in the I/O dtype; weight ~ N(0, 1/taps) fp32 ([dim, width] for the causal 1-D filter,
    [dim, width, width] for the 2-D one); bias ~ N(0, 1) fp32; state ~ N(0, 1) [batch, width-1,
    dim] in the I/O dtype (the 1-D filter's carried input rows)."""
    taps = width * width if two_d else width
    wshape = (dim, width, width) if two_d else (dim, width)
    w = (_normal(seed, 9, wshape).astype(np.float64) / np.sqrt(taps)).astype(np.float32)
    return {
        "x": _normal(seed, 10, (batch, seqlen, dim), dtype),
        "weight": w,
        "bias": _normal(seed, 11, (dim,)),
        "state": _normal(seed, 12, (batch, max(width - 1, 0), dim), dtype),
    }

