"""GPU parity past 32-bit element offsets: one batch row of 524,588 steps x 4,344 channels (bf16,
2.28e9 elements and 4.6 GB per token tensor), so that every load and store of x, delta, z, y and
the gradients reaches element offsets above 2^31 and byte offsets above 2^32, and the backward's
per-tile dB/dC partial rows (272 tiles x 2 x 16 states x 524,588 steps) above 2^32 elements.

The token tensors repeat a seeded block of P = 2^26 + 3 values (workloads.generate_periodic): P
divides neither 2^31 nor 2^32, so an offset that wrapped at either would read a different value.
The oracle sees the same values through the same index map.  Checked against it: the forward on
five channels (both ends of the first tile, the middle, and the ragged last tile of 8 channels)
over the whole sequence; the backward's per-channel gradients (dx, ddelta, dz, dA, dD) on those
channels; dB on the last 48 steps over all channels (the adjoint starts at the sequence end and
dB does not involve the state) and dC on the first 48 steps (the state starts at zero there and
dC does not involve the adjoint); and the bidirectional forward at the same size, whose second
direction's delta starts 2.28e9 elements into its tensor and whose two directions' fp32 partial
rows (a direction-split launch) are added by the merge kernel, on the same five channels; the
SS2D forward on two 512 x 512 maps of 4,344 channels (its four directions' fp32 partial rows run
to 9.1e9 elements, their index maps divide by the map's side); and the causal conv1d (k = 4 +
SiLU) on the first tensor's shape."""
import sys

import numpy as np
import pytest

import workloads as W
from tests import parity as PT

pytestmark = pytest.mark.gpu

L, DIM, P, T = 524_588, 4_344, (1 << 26) + 3, 48
CH = np.array([0, 15, 2171, 4336, 4343])


def _say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_51_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def big():
    import torch
    assert L * DIM > 1 << 31
    _say("large: drawing the blocks")
    g = W.generate_periodic(L, DIM, P)
    n = L * DIM

    def tile(block):  # [1, L, DIM] on the device, flat element i = block[i % P]
        b = PT.to_dev(block, "bf16")
        return b.repeat(-(-n // P))[:n].view(1, L, DIM)

    dev = {k: tile(g[k]) for k in ("x", "z", "delta", "dy")}
    for k in ("B", "C"):
        dev[k] = PT.to_dev(g[k], "bf16")
    dev["A"], dev["D"] = PT.to_dev(g["A"], "f32"), PT.to_dev(g["D"], "f32")
    torch.cuda.synchronize()
    _say("large: device tensors ready")
    yield g, dev
    del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _host(g, key, steps, chans):
    """Values of the full [1, L, DIM] tensor ``key`` at the given steps x channels, as fp64."""
    idx = (np.asarray(steps, dtype=np.int64)[:, None] * DIM + np.asarray(chans, dtype=np.int64)[None, :]) % P
    return W.to_f64(g[key][idx], "bf16")[None]


def test_forward_past_2_31_elements(big):
    import torch
    import oracle
    import selective_state_space_51_amd as S
    g, d = big
    y = S.selscan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"])
    ys = PT.from_dev(y[0][:, torch.from_numpy(CH).cuda()])
    torch.cuda.synchronize()
    del y
    steps = np.arange(L)
    r = oracle.selscan(_host(g, "x", steps, CH), _host(g, "delta", steps, CH), g["A"][CH].astype(np.float64),
                       W.to_f64(g["B"], "bf16"), W.to_f64(g["C"], "bf16"), D=g["D"][CH].astype(np.float64),
                       z=_host(g, "z", steps, CH))
    err = PT.rel_err(ys, r[0])
    _say("large forward", dict(L=L, dim=DIM, channels=CH.tolist()), "max rel err", err)
    assert err <= PT.TOL["bf16"], err


def test_backward_past_2_32_partials(big):
    import torch
    import oracle
    import selective_state_space_51_amd as S
    from tests.test_gpu_parity import _bwd_tol
    g, d = big
    args = dict(D=d["D"], z=d["z"])
    _, ck = S.selscan_fwd_state(d["x"], d["delta"], d["A"], d["B"], d["C"], chunk_states=True, **args)
    gr = S.selscan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["dy"], ck, **args)
    torch.cuda.synchronize()
    del ck
    ch = torch.from_numpy(CH).cuda()
    got = {k: PT.from_dev(gr[k][0][:, ch]) for k in ("dx", "ddelta", "dz")}
    got.update(dA=PT.from_dev(gr["dA"][ch]), dD=PT.from_dev(gr["dD"][ch]),
               dB=PT.from_dev(gr["dB"][0, L - T:]), dC=PT.from_dev(gr["dC"][0, :T]))
    del gr
    torch.cuda.empty_cache()
    f = lambda a: W.to_f64(a, "bf16")
    A64, D64 = g["A"].astype(np.float64), g["D"].astype(np.float64)
    # per-channel gradients: the sampled channels over the whole sequence
    steps = np.arange(L)
    h = lambda k, s, c: _host(g, k, s, c)
    r = oracle.selscan_bwd(h("x", steps, CH), h("delta", steps, CH), A64[CH], f(g["B"]), f(g["C"]), h("dy", steps, CH),
                           D=D64[CH], z=h("z", steps, CH))
    ref = {k: r[k][0] for k in ("dx", "ddelta", "dz")}
    ref.update(dA=r["dA"], dD=r["dD"])
    # dB on the last T steps and dC on the first T steps, every channel
    every = np.arange(DIM)
    tail, head = np.arange(L - T, L), np.arange(T)
    rt = oracle.selscan_bwd(h("x", tail, every), h("delta", tail, every), A64, f(g["B"][:, L - T:]),
                            f(g["C"][:, L - T:]), h("dy", tail, every), D=D64, z=h("z", tail, every))
    rh = oracle.selscan_bwd(h("x", head, every), h("delta", head, every), A64, f(g["B"][:, :T]), f(g["C"][:, :T]),
                            h("dy", head, every), D=D64, z=h("z", head, every))
    ref.update(dB=rt["dB"][0], dC=rh["dC"][0])
    errs = {k: PT.rel_err(got[k], ref[k]) for k in ref}
    _say("large backward", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= _bwd_tol("bf16", k), (k, e)


def test_bidirectional_past_2_32_elements():
    import torch
    import oracle
    import selective_state_space_51_amd as S
    _say("large bidir: drawing the blocks")
    g = W.generate_periodic(L, DIM, P, ndir=2, seed=W.SEED_BASE + 71)
    n = L * DIM

    def tile(block, k=1):  # [k, 1, L, DIM] (or [1, L, DIM]) on the device, flat element i = block[i % P]
        b = PT.to_dev(block, "bf16")
        t = b.repeat(-(-k * n // P))[:k * n]
        return t.view(k, 1, L, DIM) if k > 1 else t.view(1, L, DIM)

    x, z, dl = tile(g["x"]), tile(g["z"]), tile(g["delta"], 2)
    B, C = PT.to_dev(g["B"], "bf16"), PT.to_dev(g["C"], "bf16")
    A, D = PT.to_dev(g["A"], "f32"), PT.to_dev(g["D"], "f32")
    y = S.selscan_bidir_fwd(x, dl, A, B, C, D=D, z=z)
    ys = PT.from_dev(y[0][:, torch.from_numpy(CH).cuda()])
    torch.cuda.synchronize()
    del x, z, dl, y
    torch.cuda.empty_cache()
    steps = np.arange(L)
    idx = lambda k: (k * n + steps[:, None] * DIM + CH[None, :]) % P
    dh = np.stack([W.to_f64(g["delta"][idx(k)], "bf16")[None] for k in range(2)])
    r = oracle.selscan_bidir(_host(g, "x", steps, CH), dh, g["A"][:, CH].astype(np.float64), W.to_f64(g["B"], "bf16"),
                             W.to_f64(g["C"], "bf16"), D=g["D"][:, CH].astype(np.float64), z=_host(g, "z", steps, CH))
    err = PT.rel_err(ys, r[0])
    _say("large bidir", dict(L=L, dim=DIM, channels=CH.tolist()), "max rel err", err)
    assert err <= PT.TOL["bf16"], err


def test_ss2d_past_2_33_partials():
    import torch
    import oracle
    import selective_state_space_51_amd as S
    bt, H = 2, 512
    Lm = H * H
    n = bt * Lm * DIM
    assert n > 1 << 31
    _say("large ss2d: drawing the blocks")
    g = W.generate_periodic(Lm, DIM, P, ndir=4, batch=bt, seed=W.SEED_BASE + 72)

    def tile(block, lead):
        b = PT.to_dev(block, "bf16")
        k = int(np.prod(lead))
        return b.repeat(-(-k * n // P))[:k * n].view(*lead, bt, Lm, DIM)

    x, z, dl = tile(g["x"], ()), tile(g["z"], ()), tile(g["delta"], (4,))
    B, C = PT.to_dev(g["B"], "bf16"), PT.to_dev(g["C"], "bf16")
    A, D = PT.to_dev(g["A"], "f32"), PT.to_dev(g["D"], "f32")
    y = S.ss2d_fwd(x, dl, A, B, C, H, H, D=D, z=z)
    ys = PT.from_dev(y[:, :, torch.from_numpy(CH).cuda()])
    torch.cuda.synchronize()
    del x, z, dl, y
    torch.cuda.empty_cache()
    pos = np.arange(bt * Lm)  # (batch row, pixel) flattened

    def host(block, k=0):
        idx = (k * n + pos[:, None] * DIM + CH[None, :]) % P
        return W.to_f64(block[idx], "bf16").reshape(bt, Lm, len(CH))

    dh = np.stack([host(g["delta"], k) for k in range(4)])
    r = oracle.ss2d(host(g["x"]), dh, g["A"][:, CH].astype(np.float64), W.to_f64(g["B"], "bf16"),
                    W.to_f64(g["C"], "bf16"), H, H, D=g["D"][:, CH].astype(np.float64), z=host(g["z"]))
    err = PT.rel_err(ys, r)
    _say("large ss2d", dict(batch=bt, H=H, W=H, dim=DIM, channels=CH.tolist()), "max rel err", err)
    assert err <= PT.TOL["bf16"], err


def test_causal_conv1d_past_2_31_elements(big):
    import torch
    import oracle
    import selective_state_space_51_amd as S
    g, d = big
    c = W.generate_conv(1, 1, DIM, 4, "bf16", seed=W.SEED_BASE + 73)
    w, bias = PT.to_dev(c["weight"], "f32"), PT.to_dev(c["bias"], "f32")
    out = S.causal_conv1d_fwd(d["x"], w, bias=bias, silu=True)
    os_ = PT.from_dev(out[0][:, torch.from_numpy(CH).cuda()])
    torch.cuda.synchronize()
    del out
    torch.cuda.empty_cache()
    r = oracle.causal_conv1d(_host(g, "x", np.arange(L), CH), c["weight"][CH].astype(np.float64),
                             bias=c["bias"][CH].astype(np.float64), silu=True)
    err = PT.rel_err(os_, r[0])
    _say("large conv1d", dict(L=L, dim=DIM, channels=CH.tolist()), "max rel err", err)
    assert err <= PT.TOL["bf16"], err
