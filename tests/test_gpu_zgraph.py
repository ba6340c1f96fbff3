"""HIP graph capture.  Every entry point enqueues kernels only (no allocation, copy, memset or
synchronisation inside the library), so a captured sequence of calls replays exactly: each of
several replays, with eager work and synchronisations between them, gives the eager results
bit for bit."""
import numpy as np
import pytest

import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _inputs():
    w1 = W.Workload("graph1", "selscan", 2, 700, 64, 16, "bf16", True, index=20)
    w2 = W.Workload("graph2", "ss2d", 2, 12 * 10, 40, 16, "bf16", False, H=12, W=10, index=21)
    a1, a2 = W.generate(w1, with_bias=True), W.generate(w2)
    dev = lambda a, dt="bf16": None if a is None else PT.to_dev(a, dt)
    c1 = W.generate_conv(2, 300, 48, 4, "bf16")
    c2 = W.generate_conv(2, 9 * 11, 24, 3, "bf16", two_d=True)
    return dict(
        s1=dict(x=dev(a1["x"]), delta=dev(a1["delta"]), A=dev(a1["A"], "f32"), B=dev(a1["B"]), C=dev(a1["C"]),
                D=dev(a1["D"], "f32"), z=dev(a1["z"]), delta_bias=dev(a1["delta_bias"], "f32")),
        dy1=dev(W.generate_cotangent(2, 700, 64, "bf16")),
        s2=dict(x=dev(a2["x"]), delta=dev(a2["delta"]), A=dev(a2["A"], "f32"), B=dev(a2["B"]), C=dev(a2["C"]),
                D=dev(a2["D"], "f32")),
        dy2=dev(W.generate_cotangent(2, 120, 40, "bf16")),
        c1=dict(x=dev(c1["x"]), w=dev(c1["weight"], "f32"), b=dev(c1["bias"], "f32"), st=dev(c1["state"]),
                dout=dev(W.generate_cotangent(2, 300, 48, "bf16"))),
        c2=dict(x=dev(c2["x"]), w=dev(c2["weight"], "f32"), b=dev(c2["bias"], "f32"),
                dout=dev(W.generate_cotangent(2, 99, 24, "bf16"))),
    )


def _run_all(S, i):
    """One pass over the entry points; returns every output by name."""
    out = {}
    s1 = i["s1"]
    y1, ck1 = S.selscan_scan_fwd(S.SELSCAN_OP_FWD, **s1, delta_softplus=True, chunk_states=True)
    g1 = S.selscan_scan_bwd(S.SELSCAN_OP_FWD, s1["x"], s1["delta"], s1["A"], s1["B"], s1["C"], i["dy1"], ck1,
                            D=s1["D"], z=s1["z"], delta_bias=s1["delta_bias"], delta_softplus=True)
    out["y1"] = y1
    out.update({"g1_" + k: v for k, v in g1.items()})
    s2 = i["s2"]  # a 12 x 10 map: few workgroups, so one direction per workgroup plus the merge
    y2, ck2 = S.selscan_scan_fwd(S.SELSCAN_OP_SS2D, **s2, H=12, W=10, chunk_states=True)
    g2 = S.selscan_scan_bwd(S.SELSCAN_OP_SS2D, s2["x"], s2["delta"], s2["A"], s2["B"], s2["C"], i["dy2"], ck2,
                            D=s2["D"], H=12, W=10)
    out["y2"] = y2
    out.update({"g2_" + k: v for k, v in g2.items()})
    c1, c2 = i["c1"], i["c2"]
    out["c1"] = S.causal_conv1d_fwd(c1["x"], c1["w"], bias=c1["b"], state_in=c1["st"])
    out.update({"c1b_" + k: v for k, v in S.causal_conv1d_bwd(c1["x"], c1["w"], c1["dout"], bias=c1["b"],
                                                              state_in=c1["st"], dstate=True).items()})
    out["c2"] = S.dwconv2d_fwd(c2["x"], c2["w"], 9, 11, bias=c2["b"])
    out.update({"c2b_" + k: v for k, v in S.dwconv2d_bwd(c2["x"], c2["w"], 9, 11, c2["dout"], bias=c2["b"]).items()})
    return out


def test_graph_replay_equals_eager():
    import torch
    import selective_state_space_51_amd as S
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    inp = _inputs()
    eager = {k: v.clone() for k, v in _run_all(S, inp).items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream before capture
        _run_all(S, inp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = _run_all(S, inp)
    for rep in range(3):
        for v in cap.values():
            v.fill_(float("nan"))  # eager work between replays: every output is rewritten
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(cap[k], v), (rep, k)
    del graph
    torch.cuda.synchronize()
