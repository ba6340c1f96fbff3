"""fp64 CPU oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library (``selective_state_space_51_amd``)
never does: it shares no code with the oracle and fails loudly if its own HIP
extension is missing.

The arithmetic lives in ``oracle.c`` (plain C, double precision, the
recurrence in the order the method writes it).  This module compiles it with
gcc and marshals numpy float64 arrays.  Every function here follows the
passages cited at the top of ``oracle.c``.

Pins (the tests under ``tests/test_oracle_*.py``) check these functions against
closed forms, library routines, brute force and invariants; no function here
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no GPU needed)."""
    cmd = ["gcc", *CFLAGS, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None):
    """Load liboracle.so, building it first if it is not there or is older than oracle.c."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p) or (path is None and os.path.getmtime(_SRC) > os.path.getmtime(p)):
        build(out=p)
    lib = ctypes.CDLL(p)
    dp = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_selscan.argtypes = [dp] * 8 + [ci, ci, dp, dp, dp, i64, i64, i64, i64, ci]
    lib.oracle_selscan.restype = ci
    lib.oracle_selscan_bidir.argtypes = [dp] * 8 + [ci, ci, dp, i64, i64, i64, i64, ci]
    lib.oracle_selscan_bidir.restype = ci
    lib.oracle_ss2d.argtypes = [dp] * 8 + [ci, ci, dp, i64, i64, i64, i64, i64, ci]
    lib.oracle_ss2d.restype = ci
    lib.oracle_local_ss2d.argtypes = [dp] * 8 + [ci, ci, dp, i64, i64, i64, i64, i64, i64, ci]
    lib.oracle_local_ss2d.restype = ci
    lib.oracle_selscan_bwd.argtypes = [dp] * 8 + [ci, ci] + [dp] * 11 + [i64, i64, i64, i64, ci]
    lib.oracle_selscan_bwd.restype = ci
    lib.oracle_scan_order.argtypes = [ci, ci, i64, i64, i64, i64, dp]
    lib.oracle_scan_order.restype = ci
    lib.oracle_causal_conv1d.argtypes = [dp, dp, dp, dp, dp, ci, dp, i64, i64, i64, i64]
    lib.oracle_causal_conv1d.restype = ci
    lib.oracle_dwconv2d.argtypes = [dp, dp, dp, ci, dp, i64, i64, i64, i64, i64]
    lib.oracle_dwconv2d.restype = ci
    lib.oracle_causal_conv1d_bwd.argtypes = [dp, dp, dp, dp, dp, ci, dp, dp, dp, dp, i64, i64, i64, i64]
    lib.oracle_causal_conv1d_bwd.restype = ci
    lib.oracle_dwconv2d_bwd.argtypes = [dp, dp, dp, dp, ci, dp, dp, dp, i64, i64, i64, i64, i64]
    lib.oracle_dwconv2d_bwd.restype = ci
    lib.oracle_default_threads.argtypes = []
    lib.oracle_default_threads.restype = ci
    if path is None:
        _lib = lib
    return lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return int(load().oracle_default_threads())


def selscan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, zoh=False,
            h0=None, return_h_last=False, nthreads=0, lib=None):
    """Single-direction selective scan.

    x, delta, z: [batch][L][dim]; B, C: [batch][L][N]; A: [dim][N]; D, delta_bias: [dim];
    h0: [batch][dim][N].  Returns y (and h_last [batch][dim][N] if asked).
    """
    lib = lib or load()
    x, delta, A, B, C, D, z, delta_bias, h0 = map(_f64, (x, delta, A, B, C, D, z, delta_bias, h0))
    bt, L, dim = x.shape
    N = A.shape[-1]
    assert delta.shape == x.shape and B.shape == (bt, L, N) and C.shape == (bt, L, N) and A.shape == (dim, N)
    y = np.empty_like(x)
    hl = np.empty((bt, dim, N)) if return_h_last else None
    rc = lib.oracle_selscan(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                            int(bool(delta_softplus)), int(bool(zoh)), _ptr(h0), _ptr(hl), _ptr(y),
                            bt, L, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_selscan failed")
    return (y, hl) if return_h_last else y


def selscan_bidir(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, zoh=False,
                  nthreads=0, lib=None):
    """Bidirectional scan: per-direction arrays stacked on a leading axis of 2, token order."""
    lib = lib or load()
    x, delta, A, B, C, D, z, delta_bias = map(_f64, (x, delta, A, B, C, D, z, delta_bias))
    bt, L, dim = x.shape
    N = A.shape[-1]
    assert delta.shape == (2, bt, L, dim) and B.shape == (2, bt, L, N) and A.shape == (2, dim, N)
    y = np.empty_like(x)
    rc = lib.oracle_selscan_bidir(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh)), _ptr(y),
                                  bt, L, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_selscan_bidir failed")
    return y


def ss2d(x, delta, A, B, C, H, W, D=None, z=None, delta_bias=None, delta_softplus=False, zoh=False,
         nthreads=0, lib=None):
    """SS2D four-direction scan with merge; per-direction arrays [4][...] in pixel order."""
    lib = lib or load()
    x, delta, A, B, C, D, z, delta_bias = map(_f64, (x, delta, A, B, C, D, z, delta_bias))
    bt, L, dim = x.shape
    N = A.shape[-1]
    assert L == H * W and delta.shape == (4, bt, L, dim) and B.shape == (4, bt, L, N) and A.shape == (4, dim, N)
    y = np.empty_like(x)
    rc = lib.oracle_ss2d(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                         int(bool(delta_softplus)), int(bool(zoh)), _ptr(y), bt, H, W, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_ss2d failed")
    return y


def local_ss2d(x, delta, A, B, C, H, W, window, D=None, z=None, delta_bias=None, delta_softplus=False,
               zoh=False, nthreads=0, lib=None):
    """Windowed four-direction scan with merge (square windows of side ``window``); arrays as for ss2d."""
    lib = lib or load()
    x, delta, A, B, C, D, z, delta_bias = map(_f64, (x, delta, A, B, C, D, z, delta_bias))
    bt, L, dim = x.shape
    N = A.shape[-1]
    assert L == H * W and delta.shape == (4, bt, L, dim) and B.shape == (4, bt, L, N) and A.shape == (4, dim, N)
    y = np.empty_like(x)
    rc = lib.oracle_local_ss2d(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh)), _ptr(y), bt, H, W,
                               window, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_local_ss2d failed")
    return y


def selscan_bwd(x, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None,
                zoh=False, nthreads=0, lib=None):
    """Gradients of sum(dy * selscan(...)) with respect to every input (zoh: of the
    zero-order-hold form).

    Returns a dict with dx, ddelta (with respect to the delta argument, before bias and
    softplus), dA, dB, dC, and dD / dz / ddelta_bias / dh0 for the inputs that are given.
    """
    lib = lib or load()
    x, delta, A, B, C, dy, D, z, delta_bias, h0 = map(_f64, (x, delta, A, B, C, dy, D, z, delta_bias, h0))
    bt, L, dim = x.shape
    N = A.shape[-1]
    assert delta.shape == x.shape and dy.shape == x.shape and B.shape == (bt, L, N) and A.shape == (dim, N)
    out = {"dx": np.empty_like(x), "ddelta": np.empty_like(x), "dA": np.empty((dim, N)),
           "dB": np.empty((bt, L, N)), "dC": np.empty((bt, L, N))}
    if D is not None:
        out["dD"] = np.empty(dim)
    if z is not None:
        out["dz"] = np.empty_like(x)
    if delta_bias is not None:
        out["ddelta_bias"] = np.empty(dim)
    if h0 is not None:
        out["dh0"] = np.empty((bt, dim, N))
    g = lambda k: _ptr(out.get(k))
    rc = lib.oracle_selscan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh)), _ptr(h0), _ptr(dy),
                                g("dx"),
                                g("ddelta"), g("dA"), g("dB"), g("dC"), g("dD"), g("dz"), g("ddelta_bias"),
                                g("dh0"), bt, L, dim, N, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_selscan_bwd failed")
    return out


_KIND = {"bidir": 1, "ss2d": 2, "local_ss2d": 3}


def scan_orders(kind, L, H=0, W=0, window=0, lib=None):
    """[K][L] int64: the pixel (token) direction k visits at scan step l, from the oracle's own maps."""
    lib = lib or load()
    K = 2 if kind == "bidir" else 4
    out = np.empty((K, L), dtype=np.int64)
    for k in range(K):
        if lib.oracle_scan_order(_KIND[kind], k, H, W, window, L, out[k].ctypes.data) != 0:
            raise ValueError("bad scan order arguments")
    return out


def multi_bwd(kind, x, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False, H=0, W=0,
              window=0, zoh=False, nthreads=0, lib=None):
    """Gradients of sum(dy * y) for the multi-direction scans (bidirectional, SS2D, windowed):
    y = (sum_k scatter_k(scan_k(gather_k(x), gather_k(params_k)))) * silu(z).

    Each direction is the single-direction scan on its gathered sequence, so its gradients are
    oracle_selscan_bwd's with dL/d(its output) = gather_k(dy * silu(z)); per-token gradients are
    scattered back (dx summed over the directions).  dz = dy * yp * silu'(z) with yp the merged
    output before the gate.  Per-direction arrays carry the leading direction axis."""
    lib = lib or load()
    x, delta, A, B, C, dy, D, z, delta_bias = map(_f64, (x, delta, A, B, C, dy, D, z, delta_bias))
    bt, L, dim = x.shape
    orders = scan_orders(kind, L, H, W, window, lib=lib)
    K = orders.shape[0]
    if z is not None:
        sg = 1.0 / (1.0 + np.exp(-z))
        dyp = dy * z * sg
        if kind == "bidir":
            yp = selscan_bidir(x, delta, A, B, C, D=D, delta_bias=delta_bias, delta_softplus=delta_softplus,
                               zoh=zoh, nthreads=nthreads, lib=lib)
        elif kind == "ss2d":
            yp = ss2d(x, delta, A, B, C, H, W, D=D, delta_bias=delta_bias, delta_softplus=delta_softplus,
                      zoh=zoh, nthreads=nthreads, lib=lib)
        else:
            yp = local_ss2d(x, delta, A, B, C, H, W, window, D=D, delta_bias=delta_bias,
                            delta_softplus=delta_softplus, zoh=zoh, nthreads=nthreads, lib=lib)
    else:
        dyp = dy
    out = {"dx": np.zeros_like(x), "ddelta": np.zeros_like(delta), "dA": np.zeros_like(A), "dB": np.zeros_like(B),
           "dC": np.zeros_like(C)}
    if D is not None:
        out["dD"] = np.zeros_like(D)
    if delta_bias is not None:
        out["ddelta_bias"] = np.zeros_like(delta_bias)
    for k in range(K):
        o = orders[k]
        g = selscan_bwd(x[:, o], delta[k][:, o], A[k], B[k][:, o], C[k][:, o], dyp[:, o],
                        D=None if D is None else D[k], delta_bias=None if delta_bias is None else delta_bias[k],
                        delta_softplus=delta_softplus, zoh=zoh, nthreads=nthreads, lib=lib)
        out["dx"][:, o] += g["dx"]
        out["ddelta"][k][:, o] = g["ddelta"]
        out["dB"][k][:, o] = g["dB"]
        out["dC"][k][:, o] = g["dC"]
        out["dA"][k] = g["dA"]
        if D is not None:
            out["dD"][k] = g["dD"]
        if delta_bias is not None:
            out["ddelta_bias"][k] = g["ddelta_bias"]
    if z is not None:
        out["dz"] = dy * yp * sg * (1.0 + z * (1.0 - sg))
    return out


def ordered_scan(x, delta, A, B, C, orders, D=None, z=None, delta_bias=None, delta_softplus=False, zoh=False,
                 nthreads=0, lib=None):
    """Scans along explicit visiting orders, merged: y = (sum_k scatter_k(scan(gather_k(...)))) * silu(z).

    orders[k][l] is the token direction k visits at step l (each a permutation of range(L));
    per-direction arrays carry a leading axis of len(orders), in token order.  Each direction is
    oracle_selscan on its gathered sequence (no gate); the gate multiplies the merged sum.  This
    is the definition the fixed orders (bidirectional, SS2D, windowed) instantiate."""
    lib = lib or load()
    x, delta, A, B, C, D, z, delta_bias = map(_f64, (x, delta, A, B, C, D, z, delta_bias))
    out = np.zeros_like(x)
    for k, o in enumerate(orders):
        o = np.asarray(o, dtype=np.int64)
        yk = selscan(x[:, o], delta[k][:, o], A[k], B[k][:, o], C[k][:, o], D=None if D is None else D[k],
                     delta_bias=None if delta_bias is None else delta_bias[k], delta_softplus=delta_softplus,
                     zoh=zoh, nthreads=nthreads, lib=lib)
        out[:, o] += yk
    if z is not None:
        out *= z / (1.0 + np.exp(-z))
    return out


def causal_conv1d(x, w, bias=None, state=None, silu=True, want_state=False, lib=None):
    """Causal depthwise 1-D convolution (+ SiLU) over [batch, L, dim]; w [dim, K]; state
    [batch, K-1, dim] (the K-1 input rows before the sequence).  Returns out, or (out, state_out)."""
    lib = lib or load()
    x, w, bias, state = map(_f64, (x, w, bias, state))
    bt, L, dim = x.shape
    K = w.shape[1]
    out = np.empty_like(x)
    st = np.empty((bt, K - 1, dim)) if want_state else None
    rc = lib.oracle_causal_conv1d(_ptr(x), _ptr(w), _ptr(bias), _ptr(state), _ptr(st), int(bool(silu)), _ptr(out),
                                  bt, L, dim, K)
    if rc != 0:
        raise ValueError("oracle_causal_conv1d: bad arguments")
    return (out, st) if want_state else out


def dwconv2d(x, w, H, W, bias=None, silu=True, lib=None):
    """Depthwise ks x ks cross-correlation (+ SiLU), zero padding (ks-1)/2, over [batch, H*W, dim]
    channels-last maps; w [dim, ks, ks]."""
    lib = lib or load()
    x, w, bias = map(_f64, (x, w, bias))
    bt, L, dim = x.shape
    assert L == H * W
    out = np.empty_like(x)
    rc = lib.oracle_dwconv2d(_ptr(x), _ptr(w), _ptr(bias), int(bool(silu)), _ptr(out), bt, H, W, dim, w.shape[-1])
    if rc != 0:
        raise ValueError("oracle_dwconv2d: bad arguments")
    return out


def causal_conv1d_bwd(x, w, dout, bias=None, state=None, silu=True, lib=None):
    """Gradients of sum(dout * causal_conv1d(x, w, bias, state, silu)): a dict with dx [batch, L,
    dim], dweight [dim, K], dbias [dim] and, when a state is given, dstate [batch, K-1, dim]."""
    lib = lib or load()
    x, w, dout, bias, state = map(_f64, (x, w, dout, bias, state))
    bt, L, dim = x.shape
    K = w.shape[1]
    g = {"dx": np.empty_like(x), "dweight": np.empty((dim, K)), "dbias": np.empty(dim)}
    if state is not None:
        g["dstate"] = np.empty((bt, K - 1, dim))
    rc = lib.oracle_causal_conv1d_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(state), _ptr(dout), int(bool(silu)),
                                      _ptr(g["dx"]), _ptr(g["dweight"]), _ptr(g["dbias"]), _ptr(g.get("dstate")),
                                      bt, L, dim, K)
    if rc != 0:
        raise ValueError("oracle_causal_conv1d_bwd: bad arguments")
    return g


def dwconv2d_bwd(x, w, H, W, dout, bias=None, silu=True, lib=None):
    """Gradients of sum(dout * dwconv2d(x, w, H, W, bias, silu)): a dict with dx [batch, H*W, dim],
    dweight [dim, ks, ks] and dbias [dim]."""
    lib = lib or load()
    x, w, dout, bias = map(_f64, (x, w, dout, bias))
    bt, L, dim = x.shape
    assert L == H * W
    g = {"dx": np.empty_like(x), "dweight": np.empty_like(w), "dbias": np.empty(dim)}
    rc = lib.oracle_dwconv2d_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(dout), int(bool(silu)), _ptr(g["dx"]),
                                 _ptr(g["dweight"]), _ptr(g["dbias"]), bt, H, W, dim, w.shape[-1])
    if rc != 0:
        raise ValueError("oracle_dwconv2d_bwd: bad arguments")
    return g
