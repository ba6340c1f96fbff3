"""Pins for the fp64 oracle: each checks it against something other than itself.

Every ``pin_*`` function takes a loaded oracle library (so the mutation test can
run the same pins against copies of the oracle with planted mistakes) and
raises AssertionError when the oracle disagrees with the closed form, library
routine, brute-force evaluation or invariant it is pinned to.

Passages behind each identity are named in each docstring:
  [MS] "Mamba Series from Selective State Spaces to Visual State Space Models"
  [LM] "从LSTM到Mamba：双向状态空间模型如何重塑视觉序列建模"
"""
from __future__ import annotations

import decimal
import math

import numpy as np
import scipy.signal

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        return float("inf")
    scale = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / scale)


def _silu_np(z):
    return z / (1.0 + np.exp(-z))


def _case(seed, bt=2, L=33, dim=5, N=4, const=False):
    r = _rng(seed)
    x = r.standard_normal((bt, L, dim))
    z = r.standard_normal((bt, L, dim))
    if const:
        dt = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), (bt, 1, dim))) * np.ones((1, L, 1))
        B = r.standard_normal((bt, 1, N)) * np.ones((1, L, 1))
        C = r.standard_normal((bt, 1, N)) * np.ones((1, L, 1))
    else:
        dt = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), (bt, L, dim)))
        B = r.standard_normal((bt, L, N))
        C = r.standard_normal((bt, L, N))
    A = -np.exp(r.uniform(-1.0, 1.5, (dim, N)))
    D = r.standard_normal(dim)
    return x, z, dt, A, B, C, D


# --------------------------------------------------------------------------- P-a
def pin_lti_convolution(lib):
    """P-a.  With delta, B, C constant in time the SSM is linear time-invariant and equals a
    causal convolution of x with K_k = sum_n C_n exp(k delta A_n) Bbar_n ([MS] "选择性 SSM 的数学形式"
    and insight 1: the LTI SSM is a global convolution; [LM] §2.1 convolution view).
    Checked for both discretisations of Bbar, with D and the gate."""
    for zoh in (False, True):
        x, z, dt, A, B, C, D = _case(11 + zoh, bt=2, L=64, dim=3, N=5, const=True)
        y = oracle.selscan(x, dt, A, B, C, D=D, z=z, zoh=zoh, lib=lib)
        ref = np.empty_like(x)
        L = x.shape[1]
        k = np.arange(L)
        for b in range(x.shape[0]):
            for d in range(x.shape[2]):
                delta = dt[b, 0, d]
                a = A[d]
                bbar = (np.expm1(delta * a) / a) * B[b, 0] if zoh else delta * B[b, 0]
                K = (C[b, 0][None, :] * np.exp(np.outer(k, delta * a)) * bbar[None, :]).sum(axis=1)
                conv = np.convolve(x[b, :, d], K)[:L]
                ref[b, :, d] = (conv + D[d] * x[b, :, d]) * _silu_np(z[b, :, d])
        assert _rel(y, ref) < 1e-12, ("lti", zoh, _rel(y, ref))


# --------------------------------------------------------------------------- P-k
def pin_zoh_euler_order(lib):
    """P-k.  The zero-order-hold input matrix ([MS] "选择性 SSM 的数学形式": (delta A)^-1 (exp(delta A) - I)
    delta B) agrees with the Euler form delta B to first order in delta A.  Checked from the Taylor
    series of (e^y - 1)/y = 1 + y/2 + y^2/6 + ..., not from the closed form: (1) one step from the
    zero state (y = C Bbar x) gives the ratio r = y_zoh / y_euler with (r - 1)/(delta A) -> 1/2
    and the remainder ((r - 1)/(delta A) - 1/2)/(delta A) -> 1/6 (to 1e-3 at |delta A| <= 2e-3);
    (2) over a 12-step sequence with constant delta the gap between the two forms is second order
    in delta: halving delta divides it by 4 (to 2 %); (3) the gap changes sign with A."""
    r_ = _rng(71)
    for a in (-0.7, -2.0, 1.3):
        for delta in (2e-3, 1e-3):
            x = np.array([[[0.8]]])
            B = np.array([[[1.7]]])
            C = np.array([[[-0.6]]])
            dt = np.array([[[delta]]])
            A = np.array([[a]])
            ye = oracle.selscan(x, dt, A, B, C, lib=lib)[0, 0, 0]
            yz = oracle.selscan(x, dt, A, B, C, zoh=True, lib=lib)[0, 0, 0]
            r = yz / ye
            y = delta * a
            assert abs((r - 1.0) / y - 0.5) < abs(y), (a, delta, r)
            assert abs(((r - 1.0) / y - 0.5) / y - 1.0 / 6.0) < 1e-3, (a, delta, r)
    x = r_.standard_normal((1, 12, 2))
    B = r_.standard_normal((1, 12, 3))
    C = r_.standard_normal((1, 12, 3))
    A = np.array([[-0.5, -1.5, -3.0], [-1.0, -2.0, -4.0]])
    gaps = []
    for delta in (1e-3, 5e-4):
        dt = np.full_like(x, delta)
        gaps.append(oracle.selscan(x, dt, A, B, C, zoh=True, lib=lib) - oracle.selscan(x, dt, A, B, C, lib=lib))
    ratio = np.abs(gaps[0]).max() / np.abs(gaps[1]).max()
    assert abs(ratio / 4.0 - 1.0) < 0.02, ratio
    # A -> -A flips the sign of the leading term delta^2 A / 2 C B x of a single step
    x, B, C, dt = np.array([[[1.0]]]), np.array([[[1.0]]]), np.array([[[1.0]]]), np.array([[[1e-3]]])
    gp = oracle.selscan(x, dt, np.array([[1.0]]), B, C, zoh=True, lib=lib) - oracle.selscan(
        x, dt, np.array([[1.0]]), B, C, lib=lib)
    gm = oracle.selscan(x, dt, np.array([[-1.0]]), B, C, zoh=True, lib=lib) - oracle.selscan(
        x, dt, np.array([[-1.0]]), B, C, lib=lib)
    assert gp[0, 0, 0] > 0 > gm[0, 0, 0], (gp, gm)


# --------------------------------------------------------------------------- P-b
def pin_delta_to_zero(lib):
    """P-b.  Abar = exp(delta A) -> 1 and Bbar -> 0 as delta -> 0 ([MS] discretisation), so
    y -> D x silu(z) and the gap shrinks linearly in delta (ratio 100 for delta 1e-6 vs 1e-8)."""
    x, z, dt, A, B, C, D = _case(21, bt=1, L=40, dim=4, N=6)
    base = D[None, None, :] * x * _silu_np(z)
    gaps = []
    for delta in (1e-6, 1e-8):
        y = oracle.selscan(x, np.full_like(x, delta), A, B, C, D=D, z=z, lib=lib)
        gaps.append(np.abs(y - base).max())
    assert gaps[1] < 1e-6, gaps
    assert abs(gaps[0] / gaps[1] / 100.0 - 1.0) < 0.02, gaps
    y0 = oracle.selscan(x, np.zeros_like(x), A, B, C, D=D, z=z, lib=lib)
    assert np.array_equal(y0, D[None, None, :] * x * (z / (1.0 + np.exp(-z)))) or _rel(y0, base) < 1e-15


# --------------------------------------------------------------------------- P-c
def pin_a_zero_prefix_sum(lib):
    """P-c.  A = 0 makes Abar = 1, so h_t = sum_{s<=t} delta_s B_s x_s (a prefix sum).  With
    dyadic delta and small-integer B, C, x, D every value is exact in binary floating
    point, so the oracle must match numpy.cumsum bit for bit."""
    r = _rng(31)
    bt, L, dim, N = 2, 50, 3, 4
    x = r.integers(-3, 4, (bt, L, dim)).astype(np.float64)
    dt = r.choice([0.25, 0.5, 0.125], (bt, L, dim))
    B = r.integers(-2, 3, (bt, L, N)).astype(np.float64)
    C = r.integers(-2, 3, (bt, L, N)).astype(np.float64)
    D = r.integers(-2, 3, dim).astype(np.float64)
    A = np.zeros((dim, N))
    y = oracle.selscan(x, dt, A, B, C, D=D, lib=lib)
    h = np.cumsum((dt * x)[:, :, :, None] * B[:, :, None, :], axis=1)  # [bt, L, dim, N]
    ref = np.einsum("btn,btdn->btd", C, h) + D[None, None, :] * x
    assert np.array_equal(y, ref), np.abs(y - ref).max()


# --------------------------------------------------------------------------- P-d
def pin_first_order_iir(lib):
    """P-d.  N = 1 and constant delta: h_t = e^{delta A} h_{t-1} + delta B_t x_t is a first-order
    IIR filter; scipy.signal.lfilter evaluates it independently."""
    r = _rng(41)
    L = 300
    x = r.standard_normal((1, L, 1))
    B = r.standard_normal((1, L, 1))
    C = r.standard_normal((1, L, 1))
    delta, a, Dd = 0.07, -0.8, 0.3
    y = oracle.selscan(x, np.full_like(x, delta), np.array([[a]]), B, C, D=np.array([Dd]), lib=lib)
    h = scipy.signal.lfilter([1.0], [1.0, -math.exp(delta * a)], delta * B[0, :, 0] * x[0, :, 0])
    ref = C[0, :, 0] * h + Dd * x[0, :, 0]
    assert _rel(y[0, :, 0], ref) < 1e-12


# --------------------------------------------------------------------------- P-e
def pin_brute_force(lib):
    """P-e.  Unrolled closed form for L <= 8, evaluated in 50-digit decimal arithmetic:
    y_t = sum_n C_t[n] sum_{s<=t} exp(A_n sum_{r=s+1..t} delta_r) delta_s B_s[n] x_s + D x_t,
    then the gate.  A different algorithm (exp of sums) from the oracle's product of exps."""
    decimal.getcontext().prec = 50
    Dec = decimal.Decimal
    for seed, L in ((51, 8), (52, 5), (53, 1)):
        x, z, dt, A, B, C, D = _case(seed, bt=1, L=L, dim=3, N=4)
        y = oracle.selscan(x, dt, A, B, C, D=D, z=z, lib=lib)
        for d in range(3):
            for t in range(L):
                acc = Dec(0)
                for n in range(4):
                    inner = Dec(0)
                    for s in range(t + 1):
                        ssum = sum((Dec(float(dt[0, q, d])) for q in range(s + 1, t + 1)), Dec(0))
                        inner += (Dec(float(A[d, n])) * ssum).exp() * Dec(float(dt[0, s, d])) * \
                            Dec(float(B[0, s, n])) * Dec(float(x[0, s, d]))
                    acc += Dec(float(C[0, t, n])) * inner
                acc += Dec(float(D[d])) * Dec(float(x[0, t, d]))
                zz = Dec(float(z[0, t, d]))
                ref = acc * zz / (1 + (-zz).exp())
                got = Dec(float(y[0, t, d]))
                assert abs(got - ref) <= Dec("1e-13") * max(abs(ref), Dec(1)), (seed, t, d, got, ref)


# --------------------------------------------------------------------------- P-f
def pin_chunk_associativity(lib):
    """P-f.  The recurrence over [0, L) equals the recurrence over [0, m) followed by
    [m, L) started from the carried state (the property the chunked parallel scan of
    [MS] insight 1 relies on), and each chunk is the affine map h -> a*h + b with
    a = exp(A * sum(delta)) and b its zero-start end state."""
    x, z, dt, A, B, C, D = _case(61, bt=2, L=90, dim=3, N=5)
    y, hl = oracle.selscan(x, dt, A, B, C, D=D, return_h_last=True, lib=lib)
    m = 37
    y1, h1 = oracle.selscan(x[:, :m], dt[:, :m], A, B[:, :m], C[:, :m], D=D, return_h_last=True, lib=lib)
    y2, h2 = oracle.selscan(x[:, m:], dt[:, m:], A, B[:, m:], C[:, m:], D=D, h0=h1, return_h_last=True, lib=lib)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(h2, hl)
    # affine composition (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2)
    _, b2 = oracle.selscan(x[:, m:], dt[:, m:], A, B[:, m:], C[:, m:], D=D, return_h_last=True, lib=lib)
    a2 = np.exp(A[None, :, :] * dt[:, m:].sum(axis=1)[:, :, None])
    assert _rel(a2 * h1 + b2, hl) < 1e-12
    r = _rng(62)
    h0 = r.standard_normal(hl.shape)
    _, hh = oracle.selscan(x[:, m:], dt[:, m:], A, B[:, m:], C[:, m:], D=D, h0=h0, return_h_last=True, lib=lib)
    assert _rel(hh, a2 * h0 + b2) < 1e-12


# --------------------------------------------------------------------------- P-g
def pin_causality(lib):
    """P-g.  A scan is causal: changing x at t0 leaves every y_t, t < t0, bit-identical."""
    x, z, dt, A, B, C, D = _case(71, bt=1, L=60, dim=4, N=4)
    y = oracle.selscan(x, dt, A, B, C, D=D, z=z, lib=lib)
    x2 = x.copy()
    x2[0, 25, :] += 1.0
    y2 = oracle.selscan(x2, dt, A, B, C, D=D, z=z, lib=lib)
    assert np.array_equal(y[:, :25], y2[:, :25])
    assert not np.array_equal(y[:, 25], y2[:, 25])


# --------------------------------------------------------------------------- P-h
def pin_linearity(lib):
    """P-h.  With delta, B, C fixed and no gate the output is linear in x ([LM] §2.1: linear
    state-space system)."""
    x, z, dt, A, B, C, D = _case(81, bt=2, L=45, dim=3, N=4)
    x2 = _rng(82).standard_normal(x.shape)
    y1 = oracle.selscan(x, dt, A, B, C, D=D, lib=lib)
    y2 = oracle.selscan(x2, dt, A, B, C, D=D, lib=lib)
    y12 = oracle.selscan(1.5 * x - 0.25 * x2, dt, A, B, C, D=D, lib=lib)
    assert _rel(y12, 1.5 * y1 - 0.25 * y2) < 1e-12


# --------------------------------------------------------------------------- softplus / bias
def pin_softplus_bias(lib):
    """delta = softplus(w + bias) ([MS] selection: delta = softplus(W x + b)); numpy.logaddexp
    evaluates softplus independently.  Also checks the large-|w| branches."""
    x, z, dt, A, B, C, D = _case(91, bt=1, L=30, dim=4, N=3)
    r = _rng(92)
    w = r.standard_normal(x.shape) * 3.0
    w[0, 3, :] = [45.0, -45.0, 700.0, -700.0]
    bias = r.standard_normal(4)
    y = oracle.selscan(x, w, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=True, lib=lib)
    ref = oracle.selscan(x, np.logaddexp(0.0, w + bias), A, B, C, D=D, z=z, lib=lib)
    assert _rel(y, ref) < 1e-12


# --------------------------------------------------------------------------- gate
def pin_gate(lib):
    """SiLU gate: y = y_pre * z * sigmoid(z) ([MS] SS2Dv0.forwardv0: z = act(z), y * z; Mamba block
    diagram: the SiLU branch multiplies the SSM output).  Large |z| exercises both sides."""
    x, z, dt, A, B, C, D = _case(101, bt=1, L=20, dim=3, N=3)
    z[0, :5, :] = np.array([60.0, -60.0, 0.0])
    ypre = oracle.selscan(x, dt, A, B, C, D=D, lib=lib)
    y = oracle.selscan(x, dt, A, B, C, D=D, z=z, lib=lib)
    sig = 0.5 * (1.0 + np.tanh(0.5 * z))  # sigmoid via tanh, an independent formula
    assert _rel(y, ypre * z * sig) < 1e-12


# --------------------------------------------------------------------------- P-i
def _bidir_case(seed, bt=2, L=23, dim=4, N=3):
    r = _rng(seed)
    x = r.standard_normal((bt, L, dim))
    z = r.standard_normal((bt, L, dim))
    dt = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), (2, bt, L, dim)))
    A = -np.exp(r.uniform(-1.0, 1.5, (2, dim, N)))
    B = r.standard_normal((2, bt, L, N))
    C = r.standard_normal((2, bt, L, N))
    D = r.standard_normal((2, dim))
    return x, z, dt, A, B, C, D


def pin_bidir(lib):
    """P-i.  [LM] §3.1: the backward branch is the forward scan applied to reverse(x) with its
    own parameters.  (1) It equals two independent 1-D oracle scans composed by hand with
    numpy flips, summed and gated.  (2) Reversing every per-token array and swapping the two
    parameter sets reverses the output.  (3) delta_bwd = 0 leaves the backward branch = D_bwd x."""
    x, z, dt, A, B, C, D = _bidir_case(111)
    y = oracle.selscan_bidir(x, dt, A, B, C, D=D, z=z, lib=lib)
    f = oracle.selscan(x, dt[0], A[0], B[0], C[0], D=D[0], lib=lib)
    rb = oracle.selscan(x[:, ::-1], dt[1][:, ::-1], A[1], B[1][:, ::-1], C[1][:, ::-1], D=D[1], lib=lib)
    assert _rel(y, (f + rb[:, ::-1]) * _silu_np(z)) < 1e-13
    ys = oracle.selscan_bidir(x[:, ::-1], dt[::-1, :, ::-1], A[::-1], B[::-1, :, ::-1], C[::-1, :, ::-1],
                              D=D[::-1], z=z[:, ::-1], lib=lib)
    assert _rel(ys[:, ::-1], y) < 1e-13
    dt0 = dt.copy()
    dt0[1] = 0.0
    y0 = oracle.selscan_bidir(x, dt0, A, B, C, D=D, z=z, lib=lib)
    assert _rel(y0, (f + D[1][None, None, :] * x) * _silu_np(z)) < 1e-13


# --------------------------------------------------------------------------- P-j
def _ss2d_case(seed, bt=2, H=5, W=7, dim=3, N=3):
    r = _rng(seed)
    L = H * W
    x = r.standard_normal((bt, L, dim))
    dt = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), (4, bt, L, dim)))
    A = -np.exp(r.uniform(-1.0, 1.5, (4, dim, N)))
    B = r.standard_normal((4, bt, L, N))
    C = r.standard_normal((4, bt, L, N))
    D = r.standard_normal((4, dim))
    return x, dt, A, B, C, D


def _cross_scan_by_coordinates(lib, x, dt, A, B, C, D, H, W):
    """Reference for the four-direction scan built from pixel coordinates, independently of the
    oracle's index arithmetic: direction 0 walks the rows top to bottom, each left to right;
    direction 1 walks the columns left to right, each top to bottom; directions 2 and 3 walk
    those two paths backwards ([MS] "关键代码": row-major and column-major flattening and their
    flips).  Each direction's 1-D scan runs on its own parameters gathered along its path, and
    its outputs are added back at the pixels they were computed for."""
    rows_first = [h * W + w for h in range(H) for w in range(W)]
    cols_first = [h * W + w for w in range(W) for h in range(H)]
    paths = (rows_first, cols_first, rows_first[::-1], cols_first[::-1])
    total = np.zeros(x.shape, dtype=np.float64)
    for k, path in enumerate(paths):
        at = np.asarray(path)
        out_k = oracle.selscan(x[:, at], dt[k][:, at], A[k], B[k][:, at], C[k][:, at], D=D[k], lib=lib)
        total[:, at] += out_k  # every path visits each pixel once
    return total


def pin_ss2d(lib):
    """P-j.  SS2D = four independent 1-D scans over permuted sequences, summed at the pixel
    they came from ([MS] cross_scan_fwd / SS2Dv0.forwardv0).  (1) The index-map oracle equals
    scans along paths built from pixel coordinates.  (2) H = 1: column-major equals row-major, so
    with tied parameter pairs SS2D = 2 x bidirectional.  (3) Transposing the map (H <-> W) and
    swapping directions 0<->1, 2<->3 transposes the output."""
    for (H, W) in ((5, 7), (4, 4), (1, 6), (6, 1)):
        x, dt, A, B, C, D = _ss2d_case(121 + H * 10 + W, H=H, W=W)
        y = oracle.ss2d(x, dt, A, B, C, H, W, D=D, lib=lib)
        ref = _cross_scan_by_coordinates(lib, x, dt, A, B, C, D, H, W)
        assert _rel(y, ref) < 1e-13, (H, W, _rel(y, ref))
    # (2)
    H, W = 1, 9
    x, dt, A, B, C, D = _ss2d_case(131, H=H, W=W)
    for k in (1, 3):
        dt[k], A[k], B[k], C[k], D[k] = dt[k - 1], A[k - 1], B[k - 1], C[k - 1], D[k - 1]
    y = oracle.ss2d(x, dt, A, B, C, H, W, D=D, lib=lib)
    yb = oracle.selscan_bidir(x, dt[[0, 2]], A[[0, 2]], B[[0, 2]], C[[0, 2]], D=D[[0, 2]], lib=lib)
    assert _rel(y, 2.0 * yb) < 1e-13
    # (3)
    H, W = 4, 6
    x, dt, A, B, C, D = _ss2d_case(141, H=H, W=W)
    y = oracle.ss2d(x, dt, A, B, C, H, W, D=D, lib=lib)

    def tr(t):  # transpose the pixel axis (axis -2) of a [..., H*W, c] array: row-major H x W -> W x H
        s = t.shape
        return t.reshape(s[:-2] + (H, W, s[-1])).swapaxes(-3, -2).reshape(s)

    perm = [1, 0, 3, 2]
    yt = oracle.ss2d(tr(x), tr(dt)[perm], A[perm], tr(B)[perm], tr(C)[perm], W, H, D=D[perm], lib=lib)
    assert _rel(yt, tr(y)) < 1e-13




# --------------------------------------------------------------------------- windowed (local) scans
def _window_orders(H, W, w):
    """Scan orders of the windowed cross-scan built with array reshapes, independently of the
    oracle's index arithmetic: cut the (H, W) pixel grid into (H/w, w, W/w, w) blocks, bring
    the two window axes in front of the two in-window axes and flatten; the transposed grid
    gives direction 1; reversals give 2 and 3.  Returns [4][L] pixel indices."""
    def blocks(grid, hh, ww):
        return grid.reshape(hh // w, w, ww // w, w).transpose(0, 2, 1, 3).reshape(-1)
    pix = np.arange(H * W).reshape(H, W)
    o0 = blocks(pix, H, W)
    o1 = blocks(pix.T.copy(), W, H)
    return np.stack([o0, o1, o0[::-1], o1[::-1]])


def pin_local_ss2d_windows(lib):
    """Windowed cross-scan ([DP] LocalMamba: scan inside windows of the image) against a
    reference that gathers each direction's sequence with the reshape-built orders, runs the
    1-D oracle on it and adds the outputs back at the pixels they came from; square and
    rectangular maps, several window sides."""
    for seed, (H, W, w) in enumerate([(6, 4, 2), (6, 6, 3), (4, 8, 4), (6, 9, 3)]):
        x, dt, A, B, C, D = _ss2d_case(500 + seed, H=H, W=W)
        y = oracle.local_ss2d(x, dt, A, B, C, H, W, w, D=D, lib=lib)
        orders = _window_orders(H, W, w)
        ref = np.zeros_like(x)
        for k in range(4):
            o = orders[k]
            yk = oracle.selscan(x[:, o], dt[k][:, o], A[k], B[k][:, o], C[k][:, o], D=D[k], lib=lib)
            ref[:, o] += yk
        assert _rel(y, ref) < 1e-13, (H, W, w)


def pin_local_ss2d_limits(lib):
    """With windows of side 1, or a single window covering a square map, the windowed cross-scan
    is the SS2D cross-scan (pinned on its own by pin_ss2d): the results must be identical."""
    for H, W, w in [(5, 7, 1), (6, 6, 6), (4, 4, 1)]:
        x, dt, A, B, C, D = _ss2d_case(600 + H + w, H=H, W=W)
        a = oracle.local_ss2d(x, dt, A, B, C, H, W, w, D=D, lib=lib)
        b = oracle.ss2d(x, dt, A, B, C, H, W, D=D, lib=lib)
        assert np.array_equal(a, b), (H, W, w)


# --------------------------------------------------------------------------- backward
def _bwd_case(seed, bt=2, L=9, dim=3, N=4, gate=True, softplus=False, bias=True, h0=True, D=True, zoh=False):
    x, z, dt, A, B, C, Dv = _case(seed, bt, L, dim, N)
    r = _rng(seed + 1000)
    delta = np.log(np.expm1(dt)) if softplus else dt
    if zoh:
        # |delta A| on both sides of the oracle's series / closed-form switch at 1/2, and the
        # special values: A = 0 (Bbar = delta B), a tiny A, a positive A
        A = -np.exp(r.uniform(-1.0, 3.5, (dim, N)))
        A[0, 0] = 0.0
        A[-1, -1] = 1e-9
        A[1 % dim, 1 % N] = 0.7
    bv = 0.1 * r.standard_normal(dim)
    if zoh:
        bv = np.abs(bv)  # delta stays positive: with these |A|, exp(delta A) > 1 would blow up
    args = dict(x=x, delta=delta, A=A, B=B, C=C, D=Dv if D else None, z=z if gate else None,
                delta_bias=bv if bias else None, delta_softplus=softplus,
                h0=r.standard_normal((bt, dim, N)) if h0 else None, zoh=zoh)
    dy = r.standard_normal((bt, L, dim))
    return args, dy


def _loss(lib, args, dy):
    a = dict(args)
    h0 = a.pop("h0")
    return float(np.sum(dy * oracle.selscan(**a, h0=h0, lib=lib)))


_GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
            "delta_bias": "ddelta_bias", "h0": "dh0"}


def pin_bwd_directional_fd(lib):
    """Reverse-mode gradients of L = sum(dy * y) against central finite differences of the
    (separately pinned) forward oracle along random directions, for every input, with and
    without gate, skip, bias, softplus and initial state.  fp64: the two agree to ~1e-9."""
    for i, kw in enumerate([dict(), dict(softplus=True), dict(gate=False, bias=False, h0=False),
                            dict(D=False, softplus=True, L=17, dim=2, N=3), dict(zoh=True),
                            dict(zoh=True, softplus=True, L=13, dim=4, N=5), dict(zoh=True, gate=False, h0=False)]):
        args, dy = _bwd_case(40 + i, **kw)
        g = oracle.selscan_bwd(dy=dy, lib=lib, **args)
        r = _rng(90 + i)
        for name, gname in _GRAD_OF.items():
            if args.get(name) is None:
                continue
            v = r.standard_normal(np.shape(args[name]))
            eps = 1e-5
            up, dn = dict(args), dict(args)
            up[name] = args[name] + eps * v
            dn[name] = args[name] - eps * v
            fd = (_loss(lib, up, dy) - _loss(lib, dn, dy)) / (2 * eps)
            an = float(np.sum(g[gname] * v))
            assert abs(fd - an) <= 1e-6 * max(abs(fd), 1.0), (kw, name, fd, an)


def pin_bwd_elementwise_fd(lib):
    """Every entry of every gradient of a tiny problem against its own central difference
    (Euler and zero-order-hold Bbar)."""
    for zoh in (False, True):
        _bwd_elementwise(lib, *_bwd_case(77 + zoh, bt=2, L=4, dim=2, N=3, softplus=True, zoh=zoh))


def pin_bwd_zoh_at_A_zero(lib):
    """With A = 0 the zero-order-hold step is the Euler step (Bbar = delta B, exp(0) = 1), so
    every gradient but dA equals the Euler backward's bit for bit; dA differs (its input term,
    delta^2 phi'(0) B x = delta^2 B x / 2, is absent from the Euler form) and is pinned by the
    finite differences."""
    args, dy = _bwd_case(5, bt=2, L=11, dim=3, N=4, softplus=True)
    args["A"] = np.zeros_like(args["A"])
    ge = oracle.selscan_bwd(dy=dy, lib=lib, **args)
    gz = oracle.selscan_bwd(dy=dy, lib=lib, **dict(args, zoh=True))
    assert set(ge) == set(gz)
    for k in ge:
        if k != "dA":
            assert np.array_equal(ge[k], gz[k]), k
    assert not np.array_equal(ge["dA"], gz["dA"])


def _bwd_elementwise(lib, args, dy):
    g = oracle.selscan_bwd(dy=dy, lib=lib, **args)
    eps = 1e-6
    for name, gname in _GRAD_OF.items():
        base = np.asarray(args[name], dtype=np.float64)
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            up, dn = dict(args), dict(args)
            a = base.copy(); a[idx] += eps; up[name] = a
            b = base.copy(); b[idx] -= eps; dn[name] = b
            fd[idx] = (_loss(lib, up, dy) - _loss(lib, dn, dy)) / (2 * eps)
        assert np.abs(fd - g[gname]).max() <= 1e-6 * max(np.abs(fd).max(), 1.0), (name, fd, g[gname])



def pin_multi_bwd_fd(lib):
    """Gradients of the bidirectional, SS2D and windowed scans against central finite
    differences of their (separately pinned) forward oracles along random directions (the SS2D
    case also with the zero-order-hold Bbar)."""
    r = _rng(321)
    for kind, H, W, w, zoh in [("bidir", 0, 0, 0, False), ("ss2d", 3, 4, 0, False), ("local_ss2d", 4, 6, 2, False),
                               ("ss2d", 4, 3, 0, True)]:
        K = 2 if kind == "bidir" else 4
        bt, L, dim, N = 2, (7 if kind == "bidir" else H * W), 3, 3
        args = dict(x=r.standard_normal((bt, L, dim)), delta=np.exp(r.uniform(-5, -1.5, (K, bt, L, dim))),
                    A=-np.exp(r.uniform(-1.0, 1.5, (K, dim, N))), B=r.standard_normal((K, bt, L, N)),
                    C=r.standard_normal((K, bt, L, N)), D=r.standard_normal((K, dim)), z=r.standard_normal((bt, L, dim)),
                    delta_bias=0.1 * r.standard_normal((K, dim)), zoh=zoh)
        dy = r.standard_normal((bt, L, dim))

        def loss(a):
            if kind == "bidir":
                y = oracle.selscan_bidir(**a, lib=lib)
            elif kind == "ss2d":
                y = oracle.ss2d(**a, H=H, W=W, lib=lib)
            else:
                y = oracle.local_ss2d(**a, H=H, W=W, window=w, lib=lib)
            return float(np.sum(dy * y))

        g = oracle.multi_bwd(kind, dy=dy, H=H, W=W, window=w, lib=lib, **args)
        for name, gname in [("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
                            ("z", "dz"), ("delta_bias", "ddelta_bias")]:
            v = r.standard_normal(np.shape(args[name]))
            up, dn = dict(args), dict(args)
            up[name] = args[name] + 1e-5 * v
            dn[name] = args[name] - 1e-5 * v
            fd = (loss(up) - loss(dn)) / 2e-5
            an = float(np.sum(g[gname] * v))
            assert abs(fd - an) <= 1e-6 * max(abs(fd), 1.0), (kind, name, fd, an)



def _video_orders(T, H, W):
    """Spatial-first (frame by frame, rows, columns) and temporal-first (each pixel through the
    frames) token orders of a T x H x W clip stored frame-major, forward and reversed."""
    sf = [t * H * W + h * W + w for t in range(T) for h in range(H) for w in range(W)]
    tf = [t * H * W + h * W + w for h in range(H) for w in range(W) for t in range(T)]
    return sf, tf


def pin_ordered_scan_maps(lib):
    """ordered_scan with orders written out from their definitions reproduces the fixed-order
    oracles: bidirectional = [identity, reversal]; SS2D on an H x W map = [row-major,
    column-major, both reversed]; and a video clip's spatial-first / temporal-first orders are
    the bidirectional scan over the clip and SS2D on a T x (H W) grid."""
    r = _rng(404)
    T, H, W, dim, N, bt = 3, 2, 4, 5, 3, 2
    L = T * H * W
    x = r.standard_normal((bt, L, dim))
    z = r.standard_normal((bt, L, dim))

    def params(K):
        return dict(delta=np.exp(r.uniform(-5, -1.5, (K, bt, L, dim))), A=-np.exp(r.uniform(-1, 1.5, (K, dim, N))),
                    B=r.standard_normal((K, bt, L, N)), C=r.standard_normal((K, bt, L, N)),
                    D=r.standard_normal((K, dim)))

    sf, tf = _video_orders(T, H, W)
    p2 = params(2)
    a = oracle.ordered_scan(x, orders=[sf, sf[::-1]], z=z, lib=lib, **p2)
    b = oracle.selscan_bidir(x, z=z, lib=lib, **p2)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    p4 = params(4)
    a = oracle.ordered_scan(x, orders=[sf, tf, sf[::-1], tf[::-1]], z=z, lib=lib, **p4)
    b = oracle.ss2d(x, H=T, W=H * W, z=z, lib=lib, **p4)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # the same on an ordinary (T H) x W map: column-major written out pixel by pixel
    H2 = T * H
    rm = [h * W + w for h in range(H2) for w in range(W)]
    cm = [h * W + w for w in range(W) for h in range(H2)]
    b = oracle.ss2d(x, H=H2, W=W, z=z, lib=lib, **p4)
    a = oracle.ordered_scan(x, orders=[rm, cm, rm[::-1], cm[::-1]], z=z, lib=lib, **p4)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)



def _silu_np(v):
    return v * (0.5 * (1.0 + np.tanh(0.5 * v)))  # sigmoid written through tanh: another route than the oracle's


def pin_conv1d_impulse(lib):
    """A unit impulse at step t0 of one channel comes out as that channel's filter reversed in
    time over steps t0 .. t0+K-1 (causal: nothing before t0), and nowhere else."""
    r = _rng(501)
    bt, L, dim, K = 2, 12, 3, 4
    w = r.standard_normal((dim, K))
    x = np.zeros((bt, L, dim))
    x[1, 5, 2] = 1.0
    out = oracle.causal_conv1d(x, w, silu=False, lib=lib)
    want = np.zeros_like(x)
    for k in range(K):
        want[1, 5 + k, 2] = w[2, K - 1 - k]
    assert np.array_equal(out, want)


def pin_conv1d_numpy(lib):
    """Against numpy's full linear convolution per channel (first L outputs), with bias and SiLU,
    for filter widths 1 .. 4."""
    r = _rng(502)
    bt, L, dim = 2, 37, 5
    x = r.standard_normal((bt, L, dim))
    for K in (1, 2, 3, 4):
        w = r.standard_normal((dim, K))
        bias = r.standard_normal(dim)
        out = oracle.causal_conv1d(x, w, bias=bias, silu=True, lib=lib)
        want = np.empty_like(x)
        for b in range(bt):
            for d in range(dim):
                want[b, :, d] = np.convolve(x[b, :, d], w[d, ::-1])[:L] + bias[d]
        assert np.allclose(out, _silu_np(want), rtol=1e-13, atol=1e-13), K


def pin_conv1d_state_split(lib):
    """Streaming: the sequence in two pieces, the first piece's last K-1 input rows carried as the
    second's state, equals the whole sequence; a state in front equals prepending its rows."""
    r = _rng(503)
    bt, L, dim, K = 2, 30, 4, 4
    x = r.standard_normal((bt, L, dim))
    w = r.standard_normal((dim, K))
    st0 = r.standard_normal((bt, K - 1, dim))
    whole, st_end = oracle.causal_conv1d(x, w, state=st0, want_state=True, lib=lib)
    for m in (0, 2, 3, 17, 30):
        a, st = oracle.causal_conv1d(x[:, :m], w, state=st0, want_state=True, lib=lib)
        b, st2 = oracle.causal_conv1d(x[:, m:], w, state=st, want_state=True, lib=lib)
        assert np.array_equal(np.concatenate([a, b], axis=1), whole), m
        assert np.array_equal(st2, st_end), m
    longer = oracle.causal_conv1d(np.concatenate([st0, x], axis=1), w, lib=lib)
    assert np.allclose(longer[:, K - 1:], whole, rtol=1e-14, atol=1e-14)
    assert np.array_equal(st_end, x[:, L - (K - 1):])


def pin_dwconv2d_scipy(lib):
    """Against scipy's 2-D cross-correlation per channel ('same' size, zero fill), with bias and
    SiLU, for kernel sizes 1, 3 and 5 on a non-square map."""
    from scipy.signal import correlate2d
    r = _rng(504)
    bt, H, W, dim = 2, 7, 9, 3
    x = r.standard_normal((bt, H * W, dim))
    for ks in (1, 3, 5):
        wt = r.standard_normal((dim, ks, ks))
        bias = r.standard_normal(dim)
        out = oracle.dwconv2d(x, wt, H, W, bias=bias, silu=True, lib=lib)
        want = np.empty((bt, H, W, dim))
        for b in range(bt):
            for d in range(dim):
                want[b, :, :, d] = correlate2d(x[b, :, d].reshape(H, W), wt[d], mode="same") + bias[d]
        assert np.allclose(out, _silu_np(want).reshape(bt, H * W, dim), rtol=1e-13, atol=1e-13), ks


def pin_dwconv2d_impulse(lib):
    """A unit impulse at pixel (h0, w0) of one channel comes out as that channel's kernel turned
    by 180 degrees, centred on (h0, w0) and cut at the map's edge."""
    r = _rng(505)
    H, W, dim, ks = 5, 6, 2, 3
    wt = r.standard_normal((dim, ks, ks))
    for (h0, w0) in ((2, 3), (0, 0), (4, 5)):
        x = np.zeros((1, H * W, dim))
        x[0, h0 * W + w0, 1] = 1.0
        out = oracle.dwconv2d(x, wt, H, W, silu=False, lib=lib).reshape(H, W, dim)
        want = np.zeros((H, W, dim))
        for i in range(ks):
            for j in range(ks):
                h, w = h0 - i + 1, w0 - j + 1
                if 0 <= h < H and 0 <= w < W:
                    want[h, w, 1] = wt[1, i, j]
        assert np.array_equal(out, want), (h0, w0)


def _fd_all(loss, args, name, eps=1e-6):
    """central difference of loss for every entry of args[name]"""
    base = np.asarray(args[name], dtype=np.float64)
    fd = np.empty_like(base)
    for idx in np.ndindex(base.shape):
        up = base.copy(); up[idx] += eps
        dn = base.copy(); dn[idx] -= eps
        fd[idx] = (loss(dict(args, **{name: up})) - loss(dict(args, **{name: dn}))) / (2 * eps)
    return fd


def pin_conv1d_bwd_fd(lib):
    """Every entry of every gradient of sum(dout * causal_conv1d(...)) against its own central
    difference of the (separately pinned) forward oracle: widths 1-4, with and without SiLU,
    bias and carried state rows."""
    r = _rng(610)
    for K in (1, 2, 3, 4):
        for silu in (False, True):
            for with_state in (False, True):
                if with_state and K == 1:
                    continue
                bt, L, dim = 2, 7, 3
                args = dict(x=r.standard_normal((bt, L, dim)), w=r.standard_normal((dim, K)),
                            bias=r.standard_normal(dim) if silu else None,
                            state=r.standard_normal((bt, K - 1, dim)) if with_state else None)
                dout = r.standard_normal((bt, L, dim))

                def loss(a):
                    y = oracle.causal_conv1d(a["x"], a["w"], bias=a["bias"], state=a["state"], silu=silu, lib=lib)
                    return float(np.sum(dout * y))

                g = oracle.causal_conv1d_bwd(dout=dout, silu=silu, lib=lib, **args)
                for name, gname in (("x", "dx"), ("w", "dweight"), ("bias", "dbias"), ("state", "dstate")):
                    if args[name] is None:
                        continue
                    fd = _fd_all(loss, args, name)
                    assert np.abs(fd - g[gname]).max() <= 1e-6 * max(np.abs(fd).max(), 1.0), (K, silu, with_state, name)
                if args["bias"] is None:  # the bias gradient is the sum of dv, given or not
                    fd = _fd_all(loss, dict(args, bias=np.zeros(dim)), "bias")
                    assert np.abs(fd - g["dbias"]).max() <= 1e-6 * max(np.abs(fd).max(), 1.0), (K, "dbias")


def pin_dwconv2d_bwd_fd(lib):
    """Every entry of every gradient of sum(dout * dwconv2d(...)) against its own central
    difference of the (separately pinned) forward oracle: kernel sizes 1, 3, 5 (5 is wider than
    the 4 x 5 map's rows), with and without SiLU and bias."""
    r = _rng(620)
    for ks in (1, 3, 5):
        for silu in (False, True):
            bt, H, W, dim = 2, 4, 5, 2
            args = dict(x=r.standard_normal((bt, H * W, dim)), w=r.standard_normal((dim, ks, ks)),
                        bias=r.standard_normal(dim) if silu else None)
            dout = r.standard_normal((bt, H * W, dim))

            def loss(a):
                return float(np.sum(dout * oracle.dwconv2d(a["x"], a["w"], H, W, bias=a["bias"], silu=silu, lib=lib)))

            g = oracle.dwconv2d_bwd(args["x"], args["w"], H, W, dout, bias=args["bias"], silu=silu, lib=lib)
            for name, gname in (("x", "dx"), ("w", "dweight"), ("bias", "dbias")):
                a = args if args[name] is not None else dict(args, bias=np.zeros(dim))
                fd = _fd_all(loss, a, name)
                assert np.abs(fd - g[gname]).max() <= 1e-6 * max(np.abs(fd).max(), 1.0), (ks, silu, name)


ALL_PINS = [
    pin_lti_convolution,
    pin_delta_to_zero,
    pin_zoh_euler_order,
    pin_a_zero_prefix_sum,
    pin_first_order_iir,
    pin_brute_force,
    pin_chunk_associativity,
    pin_causality,
    pin_linearity,
    pin_softplus_bias,
    pin_gate,
    pin_bidir,
    pin_ss2d,
    pin_local_ss2d_windows,
    pin_local_ss2d_limits,
    pin_bwd_directional_fd,
    pin_bwd_elementwise_fd,
    pin_bwd_zoh_at_A_zero,
    pin_multi_bwd_fd,
    pin_ordered_scan_maps,
    pin_conv1d_impulse,
    pin_conv1d_numpy,
    pin_conv1d_state_split,
    pin_dwconv2d_scipy,
    pin_dwconv2d_impulse,
    pin_conv1d_bwd_fd,
    pin_dwconv2d_bwd_fd,
]
