"""CPU test: the oracle against hand-derived examples in tests/golden/hand_examples.json.

The pages print no numeric worked example, so each fixture is a tiny case
whose output follows by hand from the cited formula (the derivation is stored
next to the numbers).
"""
import json
import os

import numpy as np
import pytest

import oracle

CASES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_example(case):
    c = case
    f = lambda k: None if k not in c else np.asarray(c[k], dtype=np.float64)
    bt, dim, N = c["batch"], c["dim"], c["N"]
    if c["kind"] == "selscan":
        L = c["L"]
        y = oracle.selscan(f("x").reshape(bt, L, dim), f("delta").reshape(bt, L, dim), f("A"),
                           f("B").reshape(bt, L, N), f("C").reshape(bt, L, N), D=f("D"),
                           z=None if "z" not in c else f("z").reshape(bt, L, dim), zoh=c.get("zoh", False))
    elif c["kind"] == "bidir":
        L = c["L"]
        y = oracle.selscan_bidir(f("x").reshape(bt, L, dim), f("delta").reshape(2, bt, L, dim), f("A"),
                                 f("B").reshape(2, bt, L, N), f("C").reshape(2, bt, L, N), D=f("D"))
    else:
        H, W = c["H"], c["W"]
        L = H * W
        y = oracle.ss2d(f("x").reshape(bt, L, dim), f("delta").reshape(4, bt, L, dim), f("A"),
                        f("B").reshape(4, bt, L, N), f("C").reshape(4, bt, L, N), H, W, D=f("D"))
    ref = f("y").reshape(y.shape)
    assert np.abs(y - ref).max() <= c["tol"] * max(1.0, np.abs(ref).max()), (y.ravel(), ref.ravel())
