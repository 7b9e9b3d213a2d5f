"""The oracle reproduces its frozen output on the seeded tiny layer bit for bit.

tests/golden/oracle_tiny_layer.txt is written by
tests/golden/make_oracle_regression.py, which calls only the oracle; every
element of the oracle is computed in a fixed order, so any change to its
arithmetic changes some bit here.  Rewriting the fixture goes with a change to
the oracle whose justification (the passage of the pages, or the reading of
it) is stated where the change is recorded.
"""
import os

import numpy as np

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _load():
    rows = {}
    with open(os.path.join(HERE, "golden", "oracle_tiny_layer.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


def _f32(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def test_oracle_matches_frozen_tiny_layer_output():
    g = _load()
    L = synth.make_layer("tiny", seed=0)
    c = L.cfg
    toks = (0, 7, 19, 31)
    for mode, tag in ((oracle.ACT_FLOAT, "float"), (oracle.ACT_Q8, "q8")):
        o = oracle.moe_layer(L.x_f32(), L.Wr, L.bias, L.experts, L.shared, c.wfmt, c.f, c.k, act_mode=mode,
                             tokens=np.array(toks, dtype=np.int32))
        if tag == "float":
            assert np.array_equal(o["ids"].ravel(), np.array(g["ids"], dtype=np.int32))
            assert np.array_equal(o["gates"].ravel().view(np.uint32), _f32(g["gates"]).view(np.uint32))
        for i, t in enumerate(toks):
            want = _f32(g["out_%s_%d" % (tag, t)])
            assert np.array_equal(o["out"][i].view(np.uint32), want.view(np.uint32)), (tag, t)
