"""Python binding of libselscan (argument marshalling only).

Every function here has the name of the C-ABI entry point it calls (see
include/selscan.h).  torch supplies device memory and the current stream; all
arithmetic of the scan runs in the library's HIP kernels.  If libselscan.so is
missing the import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# SELSCAN_LIB names another build of the same library (the host-sanitizer test loads one built
# with AddressSanitizer and UndefinedBehaviorSanitizer on its host code)
LIB_PATH = os.environ.get("SELSCAN_LIB") or os.path.join(_PKG, "libselscan.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "selscan.h")

SELSCAN_F32 = 0
SELSCAN_BF16 = 1
SELSCAN_FLAG_DELTA_SOFTPLUS = 1
SELSCAN_FLAG_ZOH = 2
SELSCAN_FLAG_SILU = 4
SELSCAN_OP_FWD, SELSCAN_OP_BIDIR, SELSCAN_OP_SS2D, SELSCAN_OP_LOCAL_SS2D = 0, 1, 2, 3
STATUS = {
    0: "SELSCAN_OK", 1: "SELSCAN_E_NULL", 2: "SELSCAN_E_SHAPE", 3: "SELSCAN_E_ALIGN", 4: "SELSCAN_E_ALIAS",
    5: "SELSCAN_E_UNSUPPORTED", 6: "SELSCAN_E_WORKSPACE", 7: "SELSCAN_E_HIP",
}


class SelscanError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        extra = f"; HIP: {lib.selscan_last_hip_error().decode()}" if status == 7 else ""
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_str(status)}){extra}")


def _load(path=None):
    # torch carries its own HIP runtime; load it first so that the library binds to the same
    # runtime (same soname) and torch's streams and device pointers are valid in it
    import torch  # noqa: F401
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"libselscan.so not found at {path}; build it with "
            "`python selective_state_space_51_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i64, ci, cu, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    common = [vp] * 8 + [cu, vp]
    lib.selscan_fwd.argtypes = common + [i64, i64, i64, i64, ci, vp, sz, vp]
    lib.selscan_fwd_state.argtypes = common + [vp, vp, vp, i64, i64, i64, i64, ci, vp, sz, vp]
    lib.selscan_bwd.argtypes = [vp] * 8 + [cu] + [vp] * 11 + [i64, i64, i64, i64, ci, vp, sz, vp]
    lib.selscan_bwd.restype = ci
    lib.selscan_chunk_states_bytes.argtypes = [i64, i64, i64, i64]
    lib.selscan_chunk_states_bytes.restype = sz
    lib.selscan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    lib.selscan_bwd_workspace_bytes.restype = sz
    lib.selscan_bidir_fwd.argtypes = common + [i64, i64, i64, i64, ci, vp, sz, vp]
    lib.ss2d_fwd.argtypes = common + [i64, i64, i64, i64, i64, ci, vp, sz, vp]
    lib.local_ss2d_fwd.argtypes = common + [i64, i64, i64, i64, i64, i64, ci, vp, sz, vp]
    lib.local_ss2d_fwd.restype = ci
    lib.causal_conv1d_fwd.argtypes = [vp, vp, vp, vp, vp, cu, vp, i64, i64, i64, i64, ci, vp]
    lib.causal_conv1d_fwd.restype = ci
    lib.dwconv2d_fwd.argtypes = [vp, vp, vp, cu, vp, i64, i64, i64, i64, i64, ci, vp]
    lib.dwconv2d_fwd.restype = ci
    lib.causal_conv1d_bwd.argtypes = [vp, vp, vp, vp, vp, cu, vp, vp, vp, vp, i64, i64, i64, i64, ci, vp, sz, vp]
    lib.causal_conv1d_bwd.restype = ci
    lib.causal_conv1d_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    lib.causal_conv1d_bwd_workspace_bytes.restype = sz
    lib.dwconv2d_bwd.argtypes = [vp, vp, vp, vp, cu, vp, vp, vp, i64, i64, i64, i64, i64, ci, vp, sz, vp]
    lib.dwconv2d_bwd.restype = ci
    lib.dwconv2d_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ci]
    lib.dwconv2d_bwd_workspace_bytes.restype = sz
    lib.selscan_scan_fwd.argtypes = [ci] + common + [vp, i64, i64, i64, i64, i64, i64, i64, ci, vp, sz, vp]
    lib.selscan_scan_fwd.restype = ci
    lib.selscan_scan_bwd.argtypes = [ci] + [vp] * 8 + [cu] + [vp] * 10 + [i64] * 7 + [ci, vp, sz, vp]
    lib.selscan_scan_bwd.restype = ci
    lib.selscan_scan_fwd_clocked.argtypes = [ci] + common + [vp, i64, i64, i64, i64, i64, i64, i64, ci, vp, sz, vp, vp]
    lib.selscan_scan_fwd_clocked.restype = ci
    lib.selscan_clock_stamps_bytes.argtypes = [ci, i64, i64]
    lib.selscan_clock_stamps_bytes.restype = sz
    lib.selscan_scan_fwd_noalloc.argtypes = [ci] + common + [vp, i64, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.selscan_scan_fwd_noalloc.restype = ci
    lib.selscan_scan_fwd_noalloc_max_bytes.argtypes = []
    lib.selscan_scan_fwd_noalloc_max_bytes.restype = sz
    lib.selscan_scan_chunk_states_bytes.argtypes = [ci, i64, i64, i64, i64]
    lib.selscan_scan_chunk_states_bytes.restype = sz
    lib.selscan_scan_bwd_workspace_bytes.argtypes = [ci, i64, i64, i64, i64, ci]
    lib.selscan_scan_bwd_workspace_bytes.restype = sz
    for f in (lib.selscan_fwd, lib.selscan_fwd_state, lib.selscan_bidir_fwd, lib.ss2d_fwd):
        f.restype = ci
    lib.selscan_workspace_bytes.argtypes = [ci, i64, i64, i64, i64, ci]
    lib.selscan_workspace_bytes.restype = sz
    lib.selscan_status_str.argtypes = [ci]
    lib.selscan_status_str.restype = ctypes.c_char_p
    lib.selscan_abi_version.argtypes = []
    lib.selscan_abi_version.restype = ci
    lib.selscan_last_hip_error.argtypes = []
    lib.selscan_last_hip_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def use_library(path: str):
    """Bind every function of this module to another build of the same C ABI at ``path`` (the
    diagnostic libselscan_phases.so, say) from here on; returns its ctypes handle."""
    global lib, LIB_PATH
    lib = _load(path)
    LIB_PATH = path
    return lib


def status_str(status: int) -> str:
    return lib.selscan_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib.selscan_abi_version())


def header_functions():
    """Names of the functions include/selscan.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*\**\s*(\w+)\s*\(", text, re.M)))


def selscan_workspace_bytes(op: int, batch: int, seqlen_or_hw: int, dim: int, dstate: int = 16,
                            io_dtype: int = SELSCAN_BF16) -> int:
    return int(lib.selscan_workspace_bytes(op, batch, seqlen_or_hw, dim, dstate, io_dtype))


# ------------------------------------------------------------------------------ torch side
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SELSCAN_BF16
    if t.dtype == torch.float32:
        return SELSCAN_F32
    raise TypeError(f"unsupported io dtype {t.dtype}")


def _ptr(t, name, io=None, f32=False):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if f32 and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if io is not None and t.dtype != io:
        raise TypeError(f"{name} must have the io dtype {io}")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_launch_stream(fn):
    """Run `fn` with its `stream` argument (when given) as the current stream, so that every tensor
    it allocates -- outputs, and workspaces dropped once the launch is enqueued -- belongs to the
    stream the kernels run on.  The caching allocator then reuses a dropped workspace only for work
    ordered after those kernels on that stream, never for another stream's allocation while they
    still write it."""

    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, stream=None, **kwargs)
        torch = _torch()
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(s):
            return fn(*args, stream=s, **kwargs)

    return wrapped


def _workspace(op, x, bt, L, dim, workspace):
    torch = _torch()
    need = selscan_workspace_bytes(op, bt, L, dim, 16, _dtype_code(x))
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _flags(delta_softplus, zoh=False):
    return (SELSCAN_FLAG_DELTA_SOFTPLUS if delta_softplus else 0) | (SELSCAN_FLAG_ZOH if zoh else 0)


def _check(rc, what):
    if rc != 0:
        raise SelscanError(rc, what)


def _shape_check(name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@_on_launch_stream
def selscan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, y=None,
                zoh=False, workspace=None, stream=None):
    """y = (sum_n C h + D x) * silu(z) for x, delta, z: [batch, L, dim]; B, C: [batch, L, N]; A: [dim, N]."""
    torch = _torch()
    bt, L, dim = x.shape
    N = A.shape[-1]
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, (bt, L, dim)), ("B", B, (bt, L, N)), ("C", C, (bt, L, N)),
                       ("A", A, (dim, N)), ("D", D, (dim,)), ("z", z, (bt, L, dim)),
                       ("delta_bias", delta_bias, (dim,))):
        _shape_check(n_, t_, s_)
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(SELSCAN_OP_FWD, x, bt, L, dim, workspace)
    rc = lib.selscan_fwd(_ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True), _ptr(B, "B", io),
                         _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                         _ptr(delta_bias, "delta_bias", f32=True),
                         _flags(delta_softplus, zoh), _ptr(y, "y", io),
                         bt, L, dim, N, _dtype_code(x), ws, wsb, _stream(stream))
    _check(rc, "selscan_fwd")
    return y


def selscan_chunk_states_bytes(batch: int, seqlen: int, dim: int, dstate: int = 16) -> int:
    return int(lib.selscan_chunk_states_bytes(batch, seqlen, dim, dstate))


def selscan_bwd_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int = 16,
                                io_dtype: int = SELSCAN_BF16) -> int:
    return int(lib.selscan_bwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype))


@_on_launch_stream
def selscan_fwd_state(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, y=None,
                      h0=None, h_last=None, chunk_states=None, zoh=False, workspace=None, stream=None):
    """selscan_fwd with the state carried in (h0) and out (h_last), both fp32 [batch, dim, N],
    and optionally the chunk states selscan_bwd restarts from.

    h_last=True / chunk_states=True allocate those outputs; tensors are written in place
    (h_last may be h0 itself).  Returns y, or a tuple (y, h_last, chunk_states) holding the
    outputs that were asked for."""
    torch = _torch()
    bt, L, dim = x.shape
    N = A.shape[-1]
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, (bt, L, dim)), ("B", B, (bt, L, N)), ("C", C, (bt, L, N)),
                       ("A", A, (dim, N)), ("D", D, (dim,)), ("z", z, (bt, L, dim)),
                       ("delta_bias", delta_bias, (dim,)), ("h0", h0, (bt, dim, N))):
        _shape_check(n_, t_, s_)
    if h_last is True:
        h_last = torch.empty(bt, dim, N, dtype=torch.float32, device=x.device)
    _shape_check("h_last", h_last, (bt, dim, N))
    if chunk_states is True:
        chunk_states = torch.empty(max(selscan_chunk_states_bytes(bt, L, dim, N) // 4, 1), dtype=torch.float32,
                                   device=x.device)
    if chunk_states is not None and chunk_states.numel() * chunk_states.element_size() < \
            selscan_chunk_states_bytes(bt, L, dim, N):
        raise ValueError("chunk_states is smaller than selscan_chunk_states_bytes(...)")
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(SELSCAN_OP_FWD, x, bt, L, dim, workspace)
    rc = lib.selscan_fwd_state(_ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True),
                               _ptr(B, "B", io), _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                               _ptr(delta_bias, "delta_bias", f32=True),
                               _flags(delta_softplus, zoh), _ptr(y, "y", io),
                               _ptr(h0, "h0", f32=True), _ptr(h_last, "h_last", f32=True),
                               _ptr(chunk_states, "chunk_states", f32=True),
                               bt, L, dim, N, _dtype_code(x), ws, wsb, _stream(stream))
    _check(rc, "selscan_fwd_state")
    extra = tuple(t for t in (h_last, chunk_states) if t is not None)
    return (y, *extra) if extra else y


@_on_launch_stream
def selscan_bwd(x, delta, A, B, C, dy, chunk_states, D=None, z=None, delta_bias=None, delta_softplus=False,
                dh0=False, zoh=False, workspace=None, stream=None):
    """Gradients of sum(dy * y) for y = selscan_fwd(...) (zoh: of the zero-order-hold form);
    chunk_states from selscan_fwd_state on the same inputs (and the same form).  Returns a dict: dx, ddelta, dA, dB, dC, and dD / dz / ddelta_bias / dh0 for the
    inputs that were given (dh0 when asked for)."""
    torch = _torch()
    bt, L, dim = x.shape
    N = A.shape[-1]
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, (bt, L, dim)), ("B", B, (bt, L, N)), ("C", C, (bt, L, N)),
                       ("A", A, (dim, N)), ("D", D, (dim,)), ("z", z, (bt, L, dim)),
                       ("delta_bias", delta_bias, (dim,)), ("dy", dy, (bt, L, dim))):
        _shape_check(n_, t_, s_)
    f32 = dict(dtype=torch.float32, device=x.device)
    g = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x), "dA": torch.empty(dim, N, **f32),
         "dB": torch.empty(bt, L, N, dtype=io, device=x.device), "dC": torch.empty(bt, L, N, dtype=io, device=x.device)}
    if D is not None:
        g["dD"] = torch.empty(dim, **f32)
    if z is not None:
        g["dz"] = torch.empty_like(x)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty(dim, **f32)
    if dh0:
        g["dh0"] = torch.empty(bt, dim, N, **f32)
    need = selscan_bwd_workspace_bytes(bt, L, dim, N, _dtype_code(x))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() * workspace.element_size()
    p = lambda k, **kw: _ptr(g.get(k), k, **kw)
    rc = lib.selscan_bwd(_ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True), _ptr(B, "B", io),
                         _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                         _ptr(delta_bias, "delta_bias", f32=True),
                         _flags(delta_softplus, zoh),
                         _ptr(chunk_states, "chunk_states", f32=True), _ptr(dy, "dy", io),
                         p("dx", io=io), p("ddelta", io=io), p("dA", f32=True), p("dB", io=io), p("dC", io=io),
                         p("dD", f32=True), p("dz", io=io), p("ddelta_bias", f32=True), p("dh0", f32=True),
                         bt, L, dim, N, _dtype_code(x), workspace.data_ptr(), wsb, _stream(stream))
    _check(rc, "selscan_bwd")
    return g


@_on_launch_stream
def selscan_bidir_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, y=None,
                      zoh=False, workspace=None, stream=None):
    """Bidirectional scan; per-direction arrays stacked on a leading axis of 2 (token order)."""
    torch = _torch()
    bt, L, dim = x.shape
    N = A.shape[-1]
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, (2, bt, L, dim)), ("B", B, (2, bt, L, N)), ("C", C, (2, bt, L, N)),
                       ("A", A, (2, dim, N)), ("D", D, (2, dim)), ("z", z, (bt, L, dim)),
                       ("delta_bias", delta_bias, (2, dim))):
        _shape_check(n_, t_, s_)
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(SELSCAN_OP_BIDIR, x, bt, L, dim, workspace)
    rc = lib.selscan_bidir_fwd(_ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True),
                               _ptr(B, "B", io), _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                               _ptr(delta_bias, "delta_bias", f32=True),
                               _flags(delta_softplus, zoh), _ptr(y, "y", io),
                               bt, L, dim, N, _dtype_code(x), ws, wsb, _stream(stream))
    _check(rc, "selscan_bidir_fwd")
    return y


@_on_launch_stream
def ss2d_fwd(x, delta, A, B, C, H, W, D=None, z=None, delta_bias=None, delta_softplus=False, y=None,
             zoh=False, workspace=None, stream=None):
    """SS2D four-direction scan with merge; per-direction arrays [4, ...] in pixel (row-major) order."""
    torch = _torch()
    bt, L, dim = x.shape
    N = A.shape[-1]
    io = x.dtype
    if L != H * W:
        raise ValueError(f"x has {L} pixels, expected H*W = {H * W}")
    for n_, t_, s_ in (("delta", delta, (4, bt, L, dim)), ("B", B, (4, bt, L, N)), ("C", C, (4, bt, L, N)),
                       ("A", A, (4, dim, N)), ("D", D, (4, dim)), ("z", z, (bt, L, dim)),
                       ("delta_bias", delta_bias, (4, dim))):
        _shape_check(n_, t_, s_)
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(SELSCAN_OP_SS2D, x, bt, L, dim, workspace)
    rc = lib.ss2d_fwd(_ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True), _ptr(B, "B", io),
                      _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                      _ptr(delta_bias, "delta_bias", f32=True),
                      _flags(delta_softplus, zoh), _ptr(y, "y", io),
                      bt, H, W, dim, N, _dtype_code(x), ws, wsb, _stream(stream))
    _check(rc, "ss2d_fwd")
    return y


@_on_launch_stream
def local_ss2d_fwd(x, delta, A, B, C, H, W, window, D=None, z=None, delta_bias=None, delta_softplus=False, y=None,
                   zoh=False, workspace=None, stream=None):
    """Windowed four-direction cross-scan (square windows of side ``window``); arrays as for ss2d_fwd."""
    torch = _torch()
    bt, L, dim = x.shape
    N = A.shape[-1]
    io = x.dtype
    if L != H * W:
        raise ValueError(f"x has {L} pixels, expected H*W = {H * W}")
    for n_, t_, s_ in (("delta", delta, (4, bt, L, dim)), ("B", B, (4, bt, L, N)), ("C", C, (4, bt, L, N)),
                       ("A", A, (4, dim, N)), ("D", D, (4, dim)), ("z", z, (bt, L, dim)),
                       ("delta_bias", delta_bias, (4, dim))):
        _shape_check(n_, t_, s_)
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(SELSCAN_OP_LOCAL_SS2D, x, bt, L, dim, workspace)
    rc = lib.local_ss2d_fwd(_ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True), _ptr(B, "B", io),
                            _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                            _ptr(delta_bias, "delta_bias", f32=True),
                            _flags(delta_softplus, zoh), _ptr(y, "y", io),
                            bt, H, W, window, dim, N, _dtype_code(x), ws, wsb, _stream(stream))
    _check(rc, "local_ss2d_fwd")
    return y


_NDIR = {SELSCAN_OP_FWD: 1, SELSCAN_OP_BIDIR: 2, SELSCAN_OP_SS2D: 4, SELSCAN_OP_LOCAL_SS2D: 4}


def selscan_scan_chunk_states_bytes(op: int, batch: int, seqlen: int, dim: int, dstate: int = 16) -> int:
    return int(lib.selscan_scan_chunk_states_bytes(op, batch, seqlen, dim, dstate))


def selscan_scan_bwd_workspace_bytes(op: int, batch: int, seqlen: int, dim: int, dstate: int = 16,
                                     io_dtype: int = SELSCAN_BF16) -> int:
    return int(lib.selscan_scan_bwd_workspace_bytes(op, batch, seqlen, dim, dstate, io_dtype))


def _scan_shapes(op, x, A, H, W):
    bt, L, dim = x.shape
    N = A.shape[-1]
    if op not in _NDIR:
        raise ValueError(f"unknown op {op}")
    K = _NDIR[op]
    if op in (SELSCAN_OP_SS2D, SELSCAN_OP_LOCAL_SS2D) and L != H * W:
        raise ValueError(f"x has {L} pixels, expected H*W = {H * W}")
    lead = (K,) if K > 1 else ()
    return bt, L, dim, N, K, lead


@_on_launch_stream
def selscan_scan_fwd(op, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, H=0, W=0,
                     window=0, y=None, chunk_states=None, zoh=False, workspace=None, stream=None):
    """Forward of any scan order (SELSCAN_OP_*), optionally keeping the chunk states the backward
    restarts from (chunk_states=True allocates them).  Per-direction arrays carry a leading
    direction axis for the multi-direction orders.  Returns y, or (y, chunk_states)."""
    torch = _torch()
    bt, L, dim, N, K, lead = _scan_shapes(op, x, A, H, W)
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, lead + (bt, L, dim)), ("B", B, lead + (bt, L, N)),
                       ("C", C, lead + (bt, L, N)), ("A", A, lead + (dim, N)), ("D", D, lead + (dim,)),
                       ("z", z, (bt, L, dim)), ("delta_bias", delta_bias, lead + (dim,))):
        _shape_check(n_, t_, s_)
    need_cs = selscan_scan_chunk_states_bytes(op, bt, L, dim, N)
    if chunk_states is True:
        chunk_states = torch.empty(max(need_cs // 4, 1), dtype=torch.float32, device=x.device)
    if chunk_states is not None and chunk_states.numel() * chunk_states.element_size() < need_cs:
        raise ValueError("chunk_states is smaller than selscan_scan_chunk_states_bytes(...)")
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(op, x, bt, L, dim, workspace)
    rc = lib.selscan_scan_fwd(op, _ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True),
                              _ptr(B, "B", io), _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                              _ptr(delta_bias, "delta_bias", f32=True),
                              _flags(delta_softplus, zoh), _ptr(y, "y", io),
                              _ptr(chunk_states, "chunk_states", f32=True), bt, L, H, W, window, dim, N,
                              _dtype_code(x), ws, wsb, _stream(stream))
    _check(rc, "selscan_scan_fwd")
    return (y, chunk_states) if chunk_states is not None else y


def selscan_clock_stamps_bytes(op: int, batch: int, dim: int) -> int:
    return int(lib.selscan_clock_stamps_bytes(op, batch, dim))


@_on_launch_stream
def selscan_scan_fwd_clocked(op, x, delta, A, B, C, stamps, D=None, z=None, delta_bias=None, delta_softplus=False,
                             H=0, W=0, window=0, y=None, zoh=False, workspace=None, stream=None):
    """selscan_scan_fwd that also writes, per workgroup of its scan kernel, the shader-clock and
    100 MHz real-time counters at the workgroup's start and end into `stamps` (an int64 device
    tensor of at least selscan_clock_stamps_bytes(op, batch, dim) bytes).  Returns y."""
    torch = _torch()
    bt, L, dim, N, K, lead = _scan_shapes(op, x, A, H, W)
    io = x.dtype
    if stamps.dtype != torch.int64 or stamps.numel() * 8 < selscan_clock_stamps_bytes(op, bt, dim):
        raise ValueError("stamps must be int64 with selscan_clock_stamps_bytes(...) bytes")
    if y is None:
        y = torch.empty_like(x)
    ws, wsb = _workspace(op, x, bt, L, dim, workspace)
    rc = lib.selscan_scan_fwd_clocked(op, _ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True),
                                      _ptr(B, "B", io), _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                                      _ptr(delta_bias, "delta_bias", f32=True), _flags(delta_softplus, zoh),
                                      _ptr(y, "y", io), None, bt, L, H, W, window, dim, N, _dtype_code(x), ws, wsb,
                                      _ptr(stamps, "stamps"), _stream(stream))
    _check(rc, "selscan_scan_fwd_clocked")
    return y


def selscan_scan_fwd_noalloc_max_bytes() -> int:
    return int(lib.selscan_scan_fwd_noalloc_max_bytes())


@_on_launch_stream
def selscan_scan_fwd_noalloc(op, x, delta, A, B, C, y, D=None, z=None, delta_bias=None, delta_softplus=False, H=0,
                             W=0, window=0, chunk_states=None, zoh=False, stream=None):
    """selscan_scan_fwd without a workspace: the library's static device scratch holds the
    partial-sum rows, and the call allocates nothing (y, and chunk_states if wanted, are the
    caller's).  Returns y."""
    bt, L, dim, N, K, lead = _scan_shapes(op, x, A, H, W)
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, lead + (bt, L, dim)), ("B", B, lead + (bt, L, N)),
                       ("C", C, lead + (bt, L, N)), ("A", A, lead + (dim, N)), ("D", D, lead + (dim,)),
                       ("z", z, (bt, L, dim)), ("delta_bias", delta_bias, lead + (dim,)), ("y", y, (bt, L, dim))):
        _shape_check(n_, t_, s_)
    need_cs = selscan_scan_chunk_states_bytes(op, bt, L, dim, N)
    if chunk_states is not None and chunk_states.numel() * chunk_states.element_size() < need_cs:
        raise ValueError("chunk_states is smaller than selscan_scan_chunk_states_bytes(...)")
    rc = lib.selscan_scan_fwd_noalloc(op, _ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True),
                                      _ptr(B, "B", io), _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                                      _ptr(delta_bias, "delta_bias", f32=True),
                                      _flags(delta_softplus, zoh), _ptr(y, "y", io),
                                      _ptr(chunk_states, "chunk_states", f32=True), bt, L, H, W, window, dim, N,
                                      _dtype_code(x), _stream(stream))
    _check(rc, "selscan_scan_fwd_noalloc")
    return y


@_on_launch_stream
def selscan_scan_bwd(op, x, delta, A, B, C, dy, chunk_states, D=None, z=None, delta_bias=None,
                     delta_softplus=False, H=0, W=0, window=0, zoh=False, workspace=None, stream=None, grads=None):
    """Gradients of sum(dy * y) for y = selscan_scan_fwd(op, ...) with chunk_states from that call
    (zoh: of the zero-order-hold form, as the forward was run).
    Returns a dict: dx, ddelta, dA, dB, dC, and dD / dz / ddelta_bias for the inputs that were given;
    per-direction gradients carry the leading direction axis.  ``grads``: a dict of the same
    keys, shapes and dtypes to write into instead of allocating."""
    torch = _torch()
    bt, L, dim, N, K, lead = _scan_shapes(op, x, A, H, W)
    io = x.dtype
    for n_, t_, s_ in (("delta", delta, lead + (bt, L, dim)), ("B", B, lead + (bt, L, N)),
                       ("C", C, lead + (bt, L, N)), ("A", A, lead + (dim, N)), ("D", D, lead + (dim,)),
                       ("z", z, (bt, L, dim)), ("delta_bias", delta_bias, lead + (dim,)),
                       ("dy", dy, (bt, L, dim))):
        _shape_check(n_, t_, s_)
    f32 = torch.float32
    spec = {"dx": ((bt, L, dim), io), "ddelta": (lead + (bt, L, dim), io), "dA": (lead + (dim, N), f32),
            "dB": (lead + (bt, L, N), io), "dC": (lead + (bt, L, N), io)}
    if D is not None:
        spec["dD"] = (lead + (dim,), f32)
    if z is not None:
        spec["dz"] = ((bt, L, dim), io)
    if delta_bias is not None:
        spec["ddelta_bias"] = (lead + (dim,), f32)
    if grads is None:
        g = {k: torch.empty(shp, dtype=dt, device=x.device) for k, (shp, dt) in spec.items()}
    else:
        if set(grads) != set(spec):
            raise ValueError(f"grads must hold exactly {sorted(spec)}")
        for k, (shp, _) in spec.items():
            _shape_check(k, grads[k], shp)
        g = grads
    need = selscan_scan_bwd_workspace_bytes(op, bt, L, dim, N, _dtype_code(x))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() * workspace.element_size()
    p = lambda k, **kw: _ptr(g.get(k), k, **kw)
    rc = lib.selscan_scan_bwd(op, _ptr(x, "x", io), _ptr(delta, "delta", io), _ptr(A, "A", f32=True),
                              _ptr(B, "B", io), _ptr(C, "C", io), _ptr(D, "D", f32=True), _ptr(z, "z", io),
                              _ptr(delta_bias, "delta_bias", f32=True),
                              _flags(delta_softplus, zoh),
                              _ptr(chunk_states, "chunk_states", f32=True), _ptr(dy, "dy", io),
                              p("dx", io=io), p("ddelta", io=io), p("dA", f32=True), p("dB", io=io), p("dC", io=io),
                              p("dD", f32=True), p("dz", io=io), p("ddelta_bias", f32=True),
                              bt, L, H, W, window, dim, N, _dtype_code(x), workspace.data_ptr(), wsb,
                              _stream(stream))
    _check(rc, "selscan_scan_bwd")
    return g


@_on_launch_stream
def causal_conv1d_fwd(x, weight, bias=None, state_in=None, state_out=None, silu=True, out=None, stream=None):
    """Causal depthwise conv1d (+ SiLU) over x [batch, L, dim]; weight [dim, width] fp32 (width <= 4).
    state_in / state_out: [batch, width-1, dim] in x's dtype (state_out=True allocates it).
    Returns out, or (out, state_out)."""
    torch = _torch()
    bt, L, dim = x.shape
    K = weight.shape[-1]
    io = x.dtype
    _shape_check("weight", weight, (dim, K))
    _shape_check("bias", bias, (dim,))
    _shape_check("state_in", state_in, (bt, K - 1, dim))
    if state_out is True:
        state_out = torch.empty(bt, K - 1, dim, dtype=io, device=x.device)
    _shape_check("state_out", state_out, (bt, K - 1, dim))
    if out is None:
        out = torch.empty_like(x)
    rc = lib.causal_conv1d_fwd(_ptr(x, "x", io), _ptr(weight, "weight", f32=True), _ptr(bias, "bias", f32=True),
                               _ptr(state_in, "state_in", io), _ptr(state_out, "state_out", io),
                               SELSCAN_FLAG_SILU if silu else 0, _ptr(out, "out", io), bt, L, dim, K, _dtype_code(x),
                               _stream(stream))
    _check(rc, "causal_conv1d_fwd")
    return (out, state_out) if state_out is not None else out


@_on_launch_stream
def dwconv2d_fwd(x, weight, H, W, bias=None, silu=True, out=None, stream=None):
    """Depthwise 3x3 conv (+ SiLU), 'same' size, over channels-last maps x [batch, H*W, dim];
    weight [dim, 3, 3] fp32."""
    torch = _torch()
    bt, L, dim = x.shape
    io = x.dtype
    if L != H * W:
        raise ValueError(f"x has {L} pixels, expected H*W = {H * W}")
    _shape_check("weight", weight, (dim, 3, 3))
    _shape_check("bias", bias, (dim,))
    if out is None:
        out = torch.empty_like(x)
    rc = lib.dwconv2d_fwd(_ptr(x, "x", io), _ptr(weight, "weight", f32=True), _ptr(bias, "bias", f32=True),
                          SELSCAN_FLAG_SILU if silu else 0, _ptr(out, "out", io), bt, H, W, dim, 3, _dtype_code(x),
                          _stream(stream))
    _check(rc, "dwconv2d_fwd")
    return out


def causal_conv1d_bwd_workspace_bytes(batch: int, seqlen: int, dim: int, width: int, io_dtype: int = SELSCAN_BF16) -> int:
    return int(lib.causal_conv1d_bwd_workspace_bytes(batch, seqlen, dim, width, io_dtype))


def dwconv2d_bwd_workspace_bytes(batch: int, H: int, W: int, dim: int, io_dtype: int = SELSCAN_BF16) -> int:
    return int(lib.dwconv2d_bwd_workspace_bytes(batch, H, W, dim, io_dtype))


@_on_launch_stream
def causal_conv1d_bwd(x, weight, dout, bias=None, state_in=None, silu=True, dstate=False, workspace=None,
                      stream=None):
    """Gradients of sum(dout * causal_conv1d_fwd(x, weight, bias, state_in, silu)): a dict with dx
    (x's dtype), dweight, dbias (fp32) and, with dstate=True, dstate [batch, width-1, dim]."""
    torch = _torch()
    bt, L, dim = x.shape
    K = weight.shape[-1]
    io = x.dtype
    _shape_check("weight", weight, (dim, K))
    _shape_check("bias", bias, (dim,))
    _shape_check("state_in", state_in, (bt, K - 1, dim))
    _shape_check("dout", dout, (bt, L, dim))
    g = {"dx": torch.empty_like(x), "dweight": torch.empty(dim, K, dtype=torch.float32, device=x.device),
         "dbias": torch.empty(dim, dtype=torch.float32, device=x.device)}
    if dstate:
        g["dstate"] = torch.empty(bt, K - 1, dim, dtype=io, device=x.device)
    need = causal_conv1d_bwd_workspace_bytes(bt, L, dim, K, _dtype_code(x))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    rc = lib.causal_conv1d_bwd(_ptr(x, "x", io), _ptr(weight, "weight", f32=True), _ptr(bias, "bias", f32=True),
                               _ptr(state_in, "state_in", io), _ptr(dout, "dout", io), SELSCAN_FLAG_SILU if silu else 0,
                               _ptr(g["dx"], "dx", io), _ptr(g["dweight"], "dweight", f32=True),
                               _ptr(g["dbias"], "dbias", f32=True), _ptr(g.get("dstate"), "dstate", io), bt, L, dim, K,
                               _dtype_code(x), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(rc, "causal_conv1d_bwd")
    return g


@_on_launch_stream
def dwconv2d_bwd(x, weight, H, W, dout, bias=None, silu=True, workspace=None, stream=None):
    """Gradients of sum(dout * dwconv2d_fwd(x, weight, H, W, bias, silu)): a dict with dx (x's dtype),
    dweight [dim, 3, 3] and dbias (fp32)."""
    torch = _torch()
    bt, L, dim = x.shape
    io = x.dtype
    if L != H * W:
        raise ValueError(f"x has {L} pixels, expected H*W = {H * W}")
    _shape_check("weight", weight, (dim, 3, 3))
    _shape_check("bias", bias, (dim,))
    _shape_check("dout", dout, (bt, L, dim))
    g = {"dx": torch.empty_like(x), "dweight": torch.empty(dim, 3, 3, dtype=torch.float32, device=x.device),
         "dbias": torch.empty(dim, dtype=torch.float32, device=x.device)}
    need = dwconv2d_bwd_workspace_bytes(bt, H, W, dim, _dtype_code(x))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    rc = lib.dwconv2d_bwd(_ptr(x, "x", io), _ptr(weight, "weight", f32=True), _ptr(bias, "bias", f32=True),
                          _ptr(dout, "dout", io), SELSCAN_FLAG_SILU if silu else 0, _ptr(g["dx"], "dx", io),
                          _ptr(g["dweight"], "dweight", f32=True), _ptr(g["dbias"], "dbias", f32=True), bt, H, W, dim,
                          3, _dtype_code(x), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream(stream))
    _check(rc, "dwconv2d_bwd")
    return g
