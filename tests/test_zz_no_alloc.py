"""GPU test of selscan_scan_fwd_noalloc, through the C ABI: two calls in a row (the second on a
smaller problem) each equal selscan_scan_fwd with a workspace, for every multi-direction order and
for the single direction; and the call leaves the torch allocator's bookkeeping untouched."""
import sys

import numpy as np
import pytest

import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _inputs(kind, batch, L, dim, dtype, H=0, Wd=0, win=0, seed_index=21):
    w = W.Workload("noalloc_" + kind, kind, batch, L, dim, 16, dtype, kind in ("selscan", "bidir"), H=H, W=Wd,
                   index=seed_index, window=win)
    inp = W.generate(w)
    dev = {k: PT.to_dev(inp[k], dtype if k in ("x", "delta", "B", "C", "z") else "f32")
           for k in ("x", "delta", "A", "B", "C", "D", "z") if inp.get(k) is not None}
    return dev


@pytest.mark.parametrize("kind,dtype,shapes", [
    ("ss2d", "bf16", [dict(batch=3, L=120, H=10, Wd=12, dim=40), dict(batch=2, L=42, H=6, Wd=7, dim=24)]),
    ("local_ss2d", "f32", [dict(batch=2, L=144, H=12, Wd=12, win=3, dim=24), dict(batch=1, L=36, H=6, Wd=6, win=2, dim=8)]),
    ("bidir", "bf16", [dict(batch=4, L=300, dim=64), dict(batch=2, L=197, dim=32)]),
    ("bidir", "f32", [dict(batch=2, L=520, dim=48), dict(batch=1, L=77, dim=16)]),
    ("selscan", "bf16", [dict(batch=2, L=700, dim=64), dict(batch=1, L=100, dim=16)]),
])
def test_noalloc_equals_workspace_call(kind, dtype, shapes):
    import torch

    import selective_state_space_51_amd as S
    torch.cuda.synchronize()
    op = {"selscan": S.SELSCAN_OP_FWD, "bidir": S.SELSCAN_OP_BIDIR, "ss2d": S.SELSCAN_OP_SS2D,
          "local_ss2d": S.SELSCAN_OP_LOCAL_SS2D}[kind]
    for i, sh in enumerate(shapes):
        _say("noalloc", kind, dtype, i, sh)
        d = _inputs(kind, sh["batch"], sh["L"], sh["dim"], dtype, H=sh.get("H", 0), Wd=sh.get("Wd", 0),
                    win=sh.get("win", 0), seed_index=21 + i)
        geo = dict(H=sh.get("H", 0), W=sh.get("Wd", 0), window=sh.get("win", 0))
        args = (d["x"], d["delta"], d["A"], d["B"], d["C"])
        kw = dict(D=d["D"], z=d.get("z"), **geo)
        y_ref, ck_ref = S.selscan_scan_fwd(op, *args, chunk_states=True, **kw)
        y = torch.empty_like(d["x"])
        ck = torch.empty_like(ck_ref)
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        S.selscan_scan_fwd_noalloc(op, *args, y, chunk_states=ck, **kw)
        after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        torch.cuda.synchronize()
        assert after == before  # the binding and the library allocated nothing
        assert torch.equal(y, y_ref), float((y.float() - y_ref.float()).abs().max())
        assert torch.equal(ck, ck_ref)
        # and the result is the oracle's, to the forward's bar
        import oracle
        ref = {"selscan": oracle.selscan, "bidir": oracle.selscan_bidir}
        f = lambda t: PT.from_dev(t)
        if kind in ref:
            r = ref[kind](f(d["x"]), f(d["delta"]), f(d["A"]), f(d["B"]), f(d["C"]), D=f(d["D"]), z=f(d["z"]))
        elif kind == "ss2d":
            r = oracle.ss2d(f(d["x"]), f(d["delta"]), f(d["A"]), f(d["B"]), f(d["C"]), geo["H"], geo["W"], D=f(d["D"]))
        else:
            r = oracle.local_ss2d(f(d["x"]), f(d["delta"]), f(d["A"]), f(d["B"]), f(d["C"]), geo["H"], geo["W"],
                                  geo["window"], D=f(d["D"]))
        err = PT.rel_err(f(y), r)
        _say("noalloc", kind, dtype, i, "max rel err", err)
        assert err <= PT.TOL[dtype], err


def test_noalloc_refuses_oversize():
    import torch

    import selective_state_space_51_amd as S
    cap = S.selscan_scan_fwd_noalloc_max_bytes()
    # batch x L x dim x 4 > cap: refused before anything is enqueued (tensors of one element
    # stand in; validation stops at the size check)
    x = torch.zeros(1, device="cuda")
    rc = S.lib.selscan_scan_fwd_noalloc(S.SELSCAN_OP_BIDIR, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                        x.data_ptr(), None, None, None, 0, x.data_ptr(), None, 1, cap // 4 // 64 + 1, 0,
                                        0, 0, 64, 16, S.SELSCAN_F32, None)
    assert rc == 6
