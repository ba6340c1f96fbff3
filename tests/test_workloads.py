"""CPU tests of the seeded input generator (no method arithmetic lives there)."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(5)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.0e38, np.inf, -np.inf], dtype=np.float32)])
    ours = W.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_shaped():
    for w in W.WORKLOADS:
        small = dict(batch=2, seqlen=min(w.seqlen, 40), dim=min(w.dim, 24))
        a = W.generate(w, **small)
        b = W.generate(w, **small)
        for k in a:
            if a[k] is None:
                assert b[k] is None
                continue
            assert np.array_equal(a[k], b[k]), (w.name, k)
        lead = (w.ndir,) if w.ndir > 1 else ()
        assert a["x"].shape == (2, small["seqlen"], small["dim"])
        assert a["delta"].shape == lead + (2, small["seqlen"], small["dim"])
        assert a["B"].shape == lead + (2, small["seqlen"], w.dstate)
        assert a["A"].shape == lead + (small["dim"], w.dstate)
        assert (a["z"] is not None) == w.gate


def test_value_ranges():
    w = W.WORKLOADS[1]
    a = W.generate(w, batch=1, seqlen=512, dim=256)
    dl = W.to_f64(a["delta"], w.dtype)
    assert dl.min() >= 1e-3 * (1 - 2 ** -8) and dl.max() <= 1e-1 * (1 + 2 ** -8)
    # log-uniform: the log is roughly uniform on [ln 1e-3, ln 1e-1]
    lg = np.log(dl)
    assert abs(lg.mean() - 0.5 * (np.log(1e-3) + np.log(1e-1))) < 0.05
    x = W.to_f64(a["x"], w.dtype)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    assert np.array_equal(a["A"][0], -np.arange(1, 17, dtype=np.float32))


def test_softplus_inputs_reproduce_delta():
    w = W.WORKLOADS[0]
    a = W.generate(w, with_w=True, with_bias=True)
    wv = W.to_f64(a["w"], w.dtype) + a["delta_bias"].astype(np.float64)[None, None, :]
    sp = np.logaddexp(0.0, wv)
    dl = W.to_f64(a["delta"], w.dtype)
    assert np.abs(sp / dl - 1).max() < 1e-4


def test_algorithmic_bytes_formula():
    w = W.WORKLOADS[2]
    # x, delta, z, y: 4 tensors of 2*65536*4096 bf16; B, C: 2*65536*16 bf16 each; A, D fp32
    tok = 2 * 65536 * 4096
    assert w.algorithmic_bytes() == 4 * tok * 2 + 2 * 2 * 65536 * 16 * 2 + (4096 * 16 + 4096) * 4
    assert w.elements == 2 * 65536 * 4096 * 16


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says why, before it
    touches a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_periodic_blocks_are_deterministic_shaped_and_distributed():
    """The inputs of the tests past 32-bit offsets: the same values on every call, the shapes the
    scan entry points take, and the distributions of the ordinary generator."""
    a = W.generate_periodic(300, 24, 5003, ndir=4, batch=2, seed=123)
    b = W.generate_periodic(300, 24, 5003, ndir=4, batch=2, seed=123)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    for k in ("x", "z", "delta", "dy"):
        assert a[k].shape == (5003,) and a[k].dtype == np.uint16, k
    assert a["B"].shape == a["C"].shape == (4, 2, 300, 16)
    assert a["A"].shape == (4, 24, 16) and np.array_equal(a["A"][1, 5], -np.arange(1, 17, dtype=np.float32))
    assert a["D"].shape == (4, 24)
    one = W.generate_periodic(300, 24, 5003)
    assert one["B"].shape == (1, 300, 16) and one["A"].shape == (24, 16) and one["D"].shape == (24,)
    d = W.to_f64(a["delta"], "bf16")
    assert d.min() >= 1e-3 * (1 - 2 ** -8) and d.max() <= 1e-1 * (1 + 2 ** -8)
    x = W.to_f64(a["x"], "bf16")
    assert abs(x.mean()) < 0.1 and abs(x.std() - 1) < 0.1
