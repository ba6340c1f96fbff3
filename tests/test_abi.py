"""CPU tests of the C ABI: the library loads, exports what include/selscan.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed: every call
here returns from validation, except one made in a child process that sees no HIP device,
whose launch the runtime rejects)."""
import ctypes
import subprocess

import pytest

import selective_state_space_51_amd as S

L = S.lib
P = 0x10000  # a fake, aligned "device" address: validation never dereferences pointers
MB = 1 << 20


def test_exports_every_declared_symbol():
    declared = S.header_functions()
    assert set(declared) == {"selscan_fwd", "selscan_fwd_state", "selscan_bidir_fwd", "ss2d_fwd",
                             "selscan_bwd", "selscan_chunk_states_bytes", "selscan_bwd_workspace_bytes",
                             "local_ss2d_fwd", "selscan_scan_fwd", "selscan_scan_bwd",
                             "selscan_scan_chunk_states_bytes", "selscan_scan_bwd_workspace_bytes",
                             "causal_conv1d_fwd", "dwconv2d_fwd", "causal_conv1d_bwd", "dwconv2d_bwd",
                             "causal_conv1d_bwd_workspace_bytes", "dwconv2d_bwd_workspace_bytes",
                             "selscan_workspace_bytes", "selscan_scan_fwd_noalloc", "selscan_scan_fwd_noalloc_max_bytes",
                             "selscan_scan_fwd_clocked", "selscan_clock_stamps_bytes",
                             "selscan_status_str", "selscan_abi_version", "selscan_last_hip_error"}
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert hasattr(L, name)


def test_diagnostic_libraries_export_their_entry_points():
    # the phase-clock build is the scan library plus two readers of its record; the production
    # library carries neither the readers nor the record
    import os
    pkg = os.path.dirname(os.path.abspath(S.__file__))
    phases = os.path.join(pkg, "libselscan_phases.so")
    ubench = os.path.join(pkg, "libselscan_ubench.so")
    nm = lambda path: {line.split()[-1] for line in subprocess.run(
        ["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout.splitlines()
        if " T " in line}
    got = nm(phases)
    assert {"selscan_bwd_phase_read", "selscan_bwd_phase_clear", "selscan_fwd_phase_read",
            "selscan_fwd_phase_clear"} <= got
    assert set(S.header_functions()) <= got
    assert not any("phase" in name for name in nm(S.LIB_PATH))
    assert {"ub_valu_launch", "ub_read_launch", "ub_copy_launch"} <= nm(ubench)


def test_version_and_status_strings():
    assert S.abi_version() == 1
    for code in range(8):
        assert S.status_str(code) and S.status_str(code) != "unknown status"
    assert S.status_str(99) == "unknown status"


def fwd(x=P, delta=P + MB, A=P + 2 * MB, B=P + 3 * MB, C=P + 4 * MB, D=None, z=None, bias=None, flags=0,
        y=P + 8 * MB, batch=1, L_=16, dim=8, N=16, dtype=S.SELSCAN_BF16, ws=None, wsb=0):
    return L.selscan_fwd(x, delta, A, B, C, D, z, bias, flags, y, batch, L_, dim, N, dtype, ws, wsb, None)


def test_null_pointers():
    for kw in ("x", "delta", "A", "B", "C", "y"):
        assert fwd(**{kw: None}) == 1, kw


def test_negative_sizes_and_empty_noop():
    assert fwd(batch=-1) == 2
    assert fwd(L_=-3) == 2
    assert fwd(dim=-1) == 2
    # any zero size is an OK no-op, even with NULL pointers
    assert fwd(L_=0, x=None, y=None) == 0
    assert fwd(batch=0) == 0
    assert fwd(dim=0) == 0
    assert L.ss2d_fwd(P, P, P, P, P, None, None, None, 0, P, 1, -1, 4, 8, 16, 1, None, 0, None) == 2


def test_unsupported():
    assert fwd(N=8) == 5
    assert fwd(dtype=7) == 5
    assert fwd(flags=4) == 5
    # SS2D pixel indices are 32-bit: a map of 2^31 pixels is refused before any other check
    assert L.ss2d_fwd(P, P, P, P, P, None, None, None, 0, P, 1, 1 << 16, 1 << 15, 8, 16, 1, None, 0, None) == 5
    # 2^31 - 1 pixels passes that check and fails the next one (every pointer here is the same)
    assert L.ss2d_fwd(P, P, P, P, P, None, None, None, 0, P, 1, (1 << 31) - 1, 1, 8, 16, 1, None, 0, None) == 4


def test_alignment():
    assert fwd(x=P + 1) == 3
    assert fwd(A=P + 2 * MB + 2) == 3
    assert fwd(dtype=S.SELSCAN_F32, delta=P + MB + 2) == 3
    assert fwd(D=P + 5 * MB + 1) == 3


def test_alias():
    assert fwd(y=P) == 4  # y == x
    assert fwd(y=P + MB + 2) == 4  # y inside delta
    assert fwd(z=P + 6 * MB, y=P + 6 * MB) == 4
    assert fwd(D=P + 8 * MB + 16, y=P + 8 * MB) == 4


def state(h0=None, h_last=None, ckpt=None, x=P, delta=P + MB, A=P + 2 * MB, B=P + 3 * MB, C=P + 4 * MB, y=P + 8 * MB,
          batch=1, L_=16, dim=8):
    return L.selscan_fwd_state(x, delta, A, B, C, None, None, None, 0, y, h0, h_last, ckpt, batch, L_, dim, 16,
                               S.SELSCAN_BF16, None, 0, None)


def test_state_arguments():
    H = P + 16 * MB  # states: 1 x 8 x 16 fp32 = 512 bytes
    assert state(h0=H + 2) == 3
    assert state(h_last=H + 1) == 3
    assert state(h0=H, h_last=H + 256) == 4  # partial overlap (exact aliasing is allowed)
    assert state(h_last=P + 16) == 4  # inside x
    assert state(h_last=P + 2 * MB) == 4  # on A
    assert state(h0=P + 8 * MB + 8) == 4  # h0 inside y
    assert state(h_last=P + 8 * MB) == 4  # h_last on y
    # empty sequence: a no-op without h_last, and only the states are checked with it
    assert state(L_=0, x=None, delta=None, A=None, B=None, C=None, y=None) == 0
    assert state(L_=0, x=None, delta=None, A=None, B=None, C=None, y=None, h_last=H + 2) == 3
    assert state(L_=0, h0=H, h_last=H + 4) == 4
    # chunk states: 1 chunk x 8 x 16 fp32 = 512 bytes
    assert state(ckpt=H + 2) == 3
    assert state(ckpt=H, h_last=H + 256) == 4
    assert state(ckpt=P + 3 * MB + 8) == 4  # inside B
    assert S.selscan_chunk_states_bytes(2, 257, 8) == 2 * 2 * 8 * 16 * 4
    assert S.selscan_chunk_states_bytes(2, 0, 8) == 0


def bwd(**kw):
    a = dict(x=P, delta=P + MB, A=P + 2 * MB, B=P + 3 * MB, C=P + 4 * MB, D=None, z=None, bias=None, flags=0,
             ck=P + 5 * MB, dy=P + 6 * MB, dx=P + 10 * MB, ddelta=P + 11 * MB, dA=P + 12 * MB, dB=P + 13 * MB,
             dC=P + 14 * MB, dD=None, dz=None, dbias=None, dh0=None, batch=1, L_=16, dim=8, N=16,
             dtype=S.SELSCAN_BF16, ws=P + 20 * MB, wsb=1 << 20)
    a.update(kw)
    return L.selscan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"], a["ck"],
                         a["dy"], a["dx"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"],
                         a["dh0"], a["batch"], a["L_"], a["dim"], a["N"], a["dtype"], a["ws"], a["wsb"], None)


def test_bwd_arguments():
    need = S.selscan_bwd_workspace_bytes(1, 16, 8)
    assert 0 < need <= 1 << 20
    assert S.selscan_bwd_workspace_bytes(0, 16, 8) == 0
    for k in ("x", "delta", "A", "B", "C", "ck", "dy", "dx", "ddelta", "dA", "dB", "dC"):
        assert bwd(**{k: None}) == 1, k
    assert bwd(batch=-1) == 2
    # SELSCAN_FLAG_ZOH (2) is accepted; SELSCAN_FLAG_SILU (4) and unknown bits are not
    assert bwd(N=8) == 5 and bwd(flags=4) == 5 and bwd(flags=8) == 5 and bwd(flags=2, N=8) == 5
    assert bwd(dtype=3) == 5
    assert bwd(dx=P + 10 * MB + 1) == 3
    assert bwd(dA=P + 12 * MB + 2) == 3
    assert bwd(ws=None) == 6 and bwd(wsb=need - 4) == 6
    assert bwd(dx=P + 16) == 4  # output on an input
    assert bwd(dB=P + 10 * MB + 64) == 4  # two outputs overlap
    assert bwd(ws=P + 11 * MB) == 4  # workspace on an output
    assert bwd(dh0=P + 6 * MB + 4) == 4  # on dy
    # empty problems: nothing to do, or only dA (zeros) with seqlen 0
    assert bwd(batch=0, x=None, dA=None) == 0
    assert bwd(L_=0, dA=None) == 1


def scan_fwd(**kw):
    a = dict(op=S.SELSCAN_OP_BIDIR, x=P, delta=P + MB, A=P + 2 * MB, B=P + 3 * MB, C=P + 4 * MB, D=None, z=None,
             bias=None, flags=0, y=P + 8 * MB, ck=None, batch=1, L_=16, H=0, W=0, win=0, dim=8, N=16,
             dtype=S.SELSCAN_BF16, ws=P + 20 * MB, wsb=1 << 20)
    a.update(kw)
    return L.selscan_scan_fwd(a["op"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                              a["flags"], a["y"], a["ck"], a["batch"], a["L_"], a["H"], a["W"], a["win"], a["dim"],
                              a["N"], a["dtype"], a["ws"], a["wsb"], None)


def test_scan_fwd_arguments():
    """Every call here fails a host-side check (none reaches a launch)."""
    assert scan_fwd(op=7) == 5
    assert scan_fwd(op=S.SELSCAN_OP_SS2D, H=3, W=4) == 2          # 16 tokens, not 3 x 4
    assert scan_fwd(op=S.SELSCAN_OP_SS2D, H=-4, W=-4) == 2
    assert scan_fwd(op=S.SELSCAN_OP_LOCAL_SS2D, H=4, W=4, win=3) == 2
    assert scan_fwd(op=S.SELSCAN_OP_SS2D, H=4, W=4, ws=None) == 6  # shapes accepted: stops at the workspace
    # chunk states hold one block per direction: two blocks of 512 bytes for the bidirectional scan
    assert scan_fwd(ck=P + MB - 600) == 4          # the second block reaches into delta
    assert scan_fwd(ck=P + 8 * MB + 100) == 4      # on y
    assert scan_fwd(ck=P + 20 * MB + 2) == 3
    # a grid this small runs one direction per workgroup and writes a row set per direction (two
    # of 512 bytes): chunk states in the second one, past the one-set size, still overlap it
    assert scan_fwd(ck=P + 20 * MB + 600) == 4
    for op, K in ((S.SELSCAN_OP_FWD, 1), (S.SELSCAN_OP_BIDIR, 2), (S.SELSCAN_OP_SS2D, 4), (S.SELSCAN_OP_LOCAL_SS2D, 4)):
        assert S.selscan_scan_chunk_states_bytes(op, 2, 257, 8) == K * 2 * 2 * 8 * 16 * 4
    assert S.selscan_scan_chunk_states_bytes(9, 2, 257, 8) == 0
    assert S.selscan_scan_chunk_states_bytes(S.SELSCAN_OP_FWD, 2, 257, 8) == S.selscan_chunk_states_bytes(2, 257, 8)


def scan_bwd(**kw):
    a = dict(op=S.SELSCAN_OP_SS2D, x=P, delta=P + MB, A=P + 2 * MB, B=P + 3 * MB, C=P + 4 * MB, D=None, z=None,
             bias=None, flags=0, ck=P + 5 * MB, dy=P + 6 * MB, dx=P + 10 * MB, ddelta=P + 11 * MB, dA=P + 12 * MB,
             dB=P + 13 * MB, dC=P + 14 * MB, dD=None, dz=None, dbias=None, batch=1, L_=16, H=4, W=4, win=2, dim=8,
             N=16, dtype=S.SELSCAN_BF16, ws=P + 20 * MB, wsb=1 << 20)
    a.update(kw)
    return L.selscan_scan_bwd(a["op"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                              a["flags"], a["ck"], a["dy"], a["dx"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"],
                              a["dz"], a["dbias"], a["batch"], a["L_"], a["H"], a["W"], a["win"], a["dim"], a["N"],
                              a["dtype"], a["ws"], a["wsb"], None)


def test_scan_bwd_arguments():
    """Every call here fails a host-side check (none reaches a launch)."""
    ws = S.selscan_scan_bwd_workspace_bytes
    # per-tile dB/dC partials, dA and dD/dbias partials, and the fp32 dx and output rows: one set
    # per direction here (a grid this small runs one direction per workgroup), one set in all
    # when batch x channel tiles reaches 1024
    assert ws(S.SELSCAN_OP_SS2D, 1, 16, 8) == 8192 + 2048 + 256 + 4 * 512 + 4 * 512
    assert ws(S.SELSCAN_OP_FWD, 1, 16, 8) == S.selscan_bwd_workspace_bytes(1, 16, 8)
    assert ws(S.SELSCAN_OP_BIDIR, 1, 16, 8) == 4096 + 1024 + 256 + 2 * 512 + 2 * 512
    big = ws(S.SELSCAN_OP_BIDIR, 1024, 1, 16)  # 1024 x 1 tiles: the sequential walk, one row set
    assert big == 1024 * (2 * 2 * 16 * 4 + 2 * 16 * 16 * 4 + 2 * 16 * 2 * 4) + 2 * 1024 * 16 * 4
    assert ws(5, 1, 16, 8) == 0 and ws(S.SELSCAN_OP_SS2D, 0, 16, 8) == 0
    assert scan_bwd(op=5) == 5
    assert scan_bwd(H=2) == 2
    assert scan_bwd(op=S.SELSCAN_OP_LOCAL_SS2D, win=3) == 2
    for k in ("x", "delta", "A", "B", "C", "ck", "dy", "dx", "ddelta", "dA", "dB", "dC"):
        assert scan_bwd(**{k: None}) == 1, k
    assert scan_bwd(ws=None) == 6
    # the smallest accepted workspace is the sequential walk's (one row set)
    assert scan_bwd(wsb=8192 + 2048 + 256 + 512 + 512 - 4) == 6
    # four directions: dB is 4 x 512 bytes, so a dC 1 KiB after it overlaps
    assert scan_bwd(dC=P + 13 * MB + 1024) == 4
    assert scan_bwd(ddelta=P + 10 * MB - 512) == 4    # its third direction lands on dx (256 bytes)
    assert scan_bwd(dA=P + 5 * MB + 1536) == 4        # on the fourth block of chunk states (512 bytes each)


def test_workspace_query_and_check():
    # bidirectional and SS2D currently stage fp32 partial sums in the workspace
    need = S.selscan_workspace_bytes(S.SELSCAN_OP_BIDIR, 2, 10, 8)
    assert S.selscan_workspace_bytes(S.SELSCAN_OP_FWD, 2, 10, 8) == 0
    if need:
        rc = L.selscan_bidir_fwd(P, P + MB, P + 2 * MB, P + 3 * MB, P + 4 * MB, None, None, None, 0, P + 8 * MB,
                                 2, 10, 8, 16, 1, None, 0, None)
        assert rc == 6
        rc = L.selscan_bidir_fwd(P, P + MB, P + 2 * MB, P + 3 * MB, P + 4 * MB, None, None, None, 0, P + 8 * MB,
                                 2, 10, 8, 16, 1, P + 8 * MB, need, None)
        assert rc == 4  # workspace overlapping y


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        S.selscan_fwd(x, x, torch.zeros(8, 16), x.new_zeros(1, 4, 16), x.new_zeros(1, 4, 16), y=x.clone())


def test_python_scan_bwd_checks_given_grads():
    """selscan_scan_bwd(grads=...) must hold exactly the gradients of the given inputs, at their
    shapes; both checks come before any pointer is taken (host tensors suffice here)."""
    import torch
    bt, L, dim = 1, 4, 8
    x = torch.zeros(bt, L, dim, dtype=torch.bfloat16)
    bc = x.new_zeros(bt, L, 16)
    A = torch.zeros(dim, 16)
    good = {"dx": x.clone(), "ddelta": x.clone(), "dA": torch.zeros(dim, 16), "dB": bc.clone(), "dC": bc.clone()}
    call = lambda g: S.selscan_scan_bwd(0, x, x, A, bc, bc, x, torch.zeros(1), grads=g)
    with pytest.raises(ValueError, match="grads must hold"):
        call({k: v for k, v in good.items() if k != "dC"})
    with pytest.raises(ValueError, match="grads must hold"):
        call(dict(good, dz=x.clone()))
    with pytest.raises(ValueError, match="dB has shape"):
        call(dict(good, dB=x.clone()))


def test_local_ss2d_window_checks():
    loc = lambda H, W, w: L.local_ss2d_fwd(P, P + MB, P + 2 * MB, P + 3 * MB, P + 4 * MB, None, None, None, 0,
                                           P + 8 * MB, 1, H, W, w, 8, 16, 1, None, 0, None)
    assert loc(6, 4, 0) == 2   # no window
    assert loc(6, 4, 4) == 2   # does not divide H
    assert loc(6, 4, 3) == 2   # does not divide W
    assert loc(-1, 4, 1) == 2
    assert loc(6, 4, 2) == 6   # valid window: stops at the missing workspace
    # one fp32 row set per direction for a grid this small (split), one set from 1024 tiles up
    assert S.selscan_workspace_bytes(S.SELSCAN_OP_LOCAL_SS2D, 1, 24, 8) == 4 * 24 * 8 * 4
    assert S.selscan_workspace_bytes(S.SELSCAN_OP_SS2D, 1024, 4, 16) == 1024 * 4 * 16 * 4


def test_fast_division_identity():
    """The kernels divide pixel indices (< 2^31) by a runtime constant d with a multiply-high:
    m = ceil(2^(31+s) / d), 2^(s-1) < d <= 2^s, q = (n * m) >> (31 + s).  Check the identity
    on the host with the same integer recipe."""
    import numpy as np
    r = np.random.default_rng(3)
    ds = list(range(1, 300)) + [2 ** k for k in range(1, 16)] + [2 ** k + 1 for k in range(1, 16)] + \
        [int(v) for v in r.integers(2, 1 << 16, 200)] + [3136, 56, 49, 7, 65535, 65536]
    ns = np.concatenate([r.integers(0, 1 << 31, 4000), np.arange(0, 5000), [(1 << 31) - 1, (1 << 31) - 2]])
    for d in ds:
        if d == 1:
            continue
        s = (d - 1).bit_length()
        m = ((1 << (31 + s)) + d - 1) // d
        assert m < (1 << 32)
        q = [(int(n) * m) >> 32 >> (s - 1) for n in ns]
        assert q == [int(n) // d for n in ns], d


def conv1d(**kw):
    a = dict(x=P, w=P + MB, bias=None, si=None, so=None, flags=4, out=P + 2 * MB, batch=1, L_=16, dim=8, K=4,
             dtype=S.SELSCAN_BF16)
    a.update(kw)
    return L.causal_conv1d_fwd(a["x"], a["w"], a["bias"], a["si"], a["so"], a["flags"], a["out"], a["batch"],
                               a["L_"], a["dim"], a["K"], a["dtype"], None)


def test_conv1d_arguments():
    """Every call here fails a host-side check or has nothing to do (none reaches a launch)."""
    assert conv1d(K=5) == 5 and conv1d(K=0) == 5
    assert conv1d(flags=2) == 5 and conv1d(dtype=2) == 5
    assert conv1d(L_=-1) == 2
    assert conv1d(x=None) == 1 and conv1d(w=None) == 1 and conv1d(out=None) == 1
    assert conv1d(x=P + 1) == 3 and conv1d(w=P + MB + 2) == 3 and conv1d(so=P + 3 * MB + 1) == 3
    assert conv1d(out=P + 100) == 4                          # on x (16 x 8 bf16 = 256 bytes)
    assert conv1d(si=P + 3 * MB, so=P + 3 * MB + 16) == 4    # state_out on state_in (3 x 8 x 2 = 48 bytes)
    assert conv1d(so=P + 2 * MB + 64) == 4                   # state_out on out
    assert conv1d(L_=0) == 0 and conv1d(batch=0) == 0 and conv1d(dim=0) == 0


def dw(**kw):
    a = dict(x=P, w=P + MB, bias=None, flags=4, out=P + 2 * MB, batch=1, H=4, W=4, dim=8, ks=3,
             dtype=S.SELSCAN_BF16)
    a.update(kw)
    return L.dwconv2d_fwd(a["x"], a["w"], a["bias"], a["flags"], a["out"], a["batch"], a["H"], a["W"], a["dim"],
                          a["ks"], a["dtype"], None)


def test_dwconv2d_arguments():
    """Every call here fails a host-side check or has nothing to do (none reaches a launch)."""
    assert dw(ks=5) == 5 and dw(ks=1) == 5 and dw(flags=1) == 5
    assert dw(H=-1) == 2
    assert dw(x=None) == 1 and dw(w=None) == 1
    assert dw(out=P + 200) == 4 and dw(out=P + MB + 16) == 4
    assert dw(x=P + 1) == 3
    assert dw(H=0) == 0 and dw(batch=0) == 0



def c1b(**kw):
    a = dict(x=P, w=P + MB, bias=None, st=None, dout=P + 2 * MB, flags=0, dx=P + 3 * MB, dw=P + 4 * MB, db=None,
             dst=None, batch=1, L_=16, dim=8, K=4, dtype=S.SELSCAN_BF16, ws=P + 8 * MB, wsb=1 << 20)
    a.update(kw)
    return L.causal_conv1d_bwd(a["x"], a["w"], a["bias"], a["st"], a["dout"], a["flags"], a["dx"], a["dw"], a["db"],
                               a["dst"], a["batch"], a["L_"], a["dim"], a["K"], a["dtype"], a["ws"], a["wsb"], None)


def test_conv1d_bwd_arguments():
    """Every call here fails a host-side check (none reaches a launch)."""
    need = S.causal_conv1d_bwd_workspace_bytes(1, 16, 8, 4)
    assert 16 * 8 * 4 <= need <= 1 << 20
    assert S.causal_conv1d_bwd_workspace_bytes(0, 16, 8, 4) == 0 and S.causal_conv1d_bwd_workspace_bytes(1, 16, 8, 5) == 0
    assert c1b(batch=-1) == 2
    assert c1b(K=5) == 5 and c1b(K=0) == 5 and c1b(flags=1) == 5 and c1b(dtype=3) == 5
    for k in ("x", "w", "dout", "dx", "dw"):
        assert c1b(**{k: None}) == 1, k
    assert c1b(dx=P + 3 * MB + 1) == 3 and c1b(dw=P + 4 * MB + 2) == 3
    assert c1b(ws=None) == 6 and c1b(wsb=need - 4) == 6
    assert c1b(dx=P + 16) == 4                    # dx on x
    assert c1b(dw=P + 3 * MB + 64) == 4           # dweight on dx
    assert c1b(ws=P + 2 * MB) == 4                # the workspace on dout
    assert c1b(dst=P + MB + 16, st=P + 5 * MB) == 4  # dstate on the filters
    assert c1b(batch=0, x=None) == 0


def d2b(**kw):
    a = dict(x=P, w=P + MB, bias=None, dout=P + 2 * MB, flags=0, dx=P + 3 * MB, dw=P + 4 * MB, db=None, batch=1, H=4,
             W=5, dim=8, ks=3, dtype=S.SELSCAN_BF16, ws=P + 8 * MB, wsb=1 << 20)
    a.update(kw)
    return L.dwconv2d_bwd(a["x"], a["w"], a["bias"], a["dout"], a["flags"], a["dx"], a["dw"], a["db"], a["batch"],
                          a["H"], a["W"], a["dim"], a["ks"], a["dtype"], a["ws"], a["wsb"], None)


def test_dwconv2d_bwd_arguments():
    """Every call here fails a host-side check (none reaches a launch)."""
    need = S.dwconv2d_bwd_workspace_bytes(1, 4, 5, 8)
    assert 20 * 8 * 4 <= need <= 1 << 20 and S.dwconv2d_bwd_workspace_bytes(1, 0, 5, 8) == 0
    assert d2b(H=-1) == 2 and d2b(ks=5) == 5 and d2b(flags=2) == 5
    for k in ("x", "w", "dout", "dx", "dw"):
        assert d2b(**{k: None}) == 1, k
    assert d2b(dx=P + 3 * MB + 1) == 3
    assert d2b(ws=None) == 6 and d2b(wsb=need - 4) == 6
    assert d2b(dx=P + 2 * MB + 16) == 4 and d2b(db=P + 3 * MB + 4) == 4
    assert d2b(dim=0) == 0


def test_bench_finds_profiled_kernels_in_library():
    """The counter records are keyed to the machine code of named kernels in the built library:
    every name bench.py asks for must be there (a rename would silently drop the traffic figure)."""
    import bench
    for ps in ("fwd", "bwd", "conv"):
        for kind in ("selscan", "bidir", "ss2d", "local_ss2d"):
            h = bench.kernel_code_hash(bench.profiled_kernels(ps, kind))
            assert not h.startswith("missing"), (ps, kind, h)
            assert len(h) == 16
    # the three-workgroup forward form of every order
    for kind in ("selscan", "bidir", "ss2d", "local_ss2d"):
        h = bench.kernel_code_hash(bench.profiled_kernels("fwd", kind, occ3=True))
        assert not h.startswith("missing"), (kind, h)


def test_scan_fwd_noalloc_arguments():
    """Host-side refusals of the no-allocation forward (none reaches a HIP call): an unknown op,
    a map that is not H x W, and a problem whose partial-sum rows exceed the static array."""
    cap = S.selscan_scan_fwd_noalloc_max_bytes()
    assert cap == 128 << 20

    def call(op=S.SELSCAN_OP_SS2D, batch=1, L_=16, H=4, W=4, dim=8):
        return L.selscan_scan_fwd_noalloc(op, P, P + MB, P + 2 * MB, P + 3 * MB, P + 4 * MB, None, None, None, 0,
                                          P + 8 * MB, None, batch, L_, H, W, 0, dim, 16, S.SELSCAN_BF16, None)
    assert call(op=9) == 5
    assert call(H=3) == 2
    # one fp32 row set of 64 x 4096 x 256 x 4 bytes = 256 MiB > 128 MiB
    assert call(batch=64, L_=4096, H=64, W=64, dim=256) == 6
    assert call(op=S.SELSCAN_OP_BIDIR, batch=64, L_=4096, H=0, W=0, dim=256) == 6


def test_clocked_forward_arguments():
    """The clocked forward refuses a NULL or misaligned stamps buffer before anything else; its size
    query counts 32 bytes per workgroup of the largest grid."""
    ck = lambda stamps, op=S.SELSCAN_OP_SS2D: L.selscan_scan_fwd_clocked(
        op, P, P + MB, P + 2 * MB, P + 3 * MB, P + 4 * MB, None, None, None, 0, P + 8 * MB, None, 1, 16, 4, 4, 0, 8,
        16, S.SELSCAN_BF16, None, 0, stamps, None)
    assert ck(None) == 1
    assert ck(P + 20 * MB + 4) == 3
    assert ck(P + 20 * MB, op=9) == 5
    assert ck(P + 20 * MB) == 6  # the SS2D call itself then stops at the missing workspace
    assert S.selscan_clock_stamps_bytes(S.SELSCAN_OP_SS2D, 2, 40) == 2 * 3 * 4 * 32
    assert S.selscan_clock_stamps_bytes(S.SELSCAN_OP_FWD, 2, 40) == 2 * 3 * 32
    assert S.selscan_clock_stamps_bytes(7, 2, 40) == 0


_NO_DEVICE_CALL = r'''
import ctypes, sys
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
    print("SKIP a device is visible")  # never launch with fake pointers where a GPU could run it
    sys.exit(0)
import selective_state_space_51_amd as S
P, MB = 0x10000, 1 << 20
rc = S.lib.selscan_fwd(P, P + MB, P + 2 * MB, P + 3 * MB, P + 4 * MB, None, None, None, 0, P + 8 * MB,
                       1, 16, 8, 16, S.SELSCAN_BF16, None, 0, None)
msg = S.lib.selscan_last_hip_error()
print("RC", rc, (msg or b"").decode())
'''


def test_hip_error_path_without_a_device():
    """Arguments that pass every host check, with no HIP device visible: the launch is rejected by
    the runtime, and the call returns SELSCAN_E_HIP with the runtime's message (the child process
    hides every device and checks that none is visible before it calls; nothing runs on a GPU)."""
    import os
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", _NO_DEVICE_CALL], capture_output=True, text=True, env=env,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))), timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    line = out.stdout.strip().splitlines()[-1]
    if line.startswith("SKIP"):
        pytest.skip(line)
    parts = line.split(" ", 2)
    assert parts[0] == "RC" and int(parts[1]) == 7, line  # SELSCAN_E_HIP
    assert len(parts) == 3 and parts[2] and parts[2] != "no error", line
    assert S.status_str(7) == "the HIP runtime rejected the kernel launch"
