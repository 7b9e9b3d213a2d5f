"""Write tests/golden/oracle_tiny_layer.txt from the oracle (and only the oracle).

The fixture freezes the oracle's output on the seeded tiny layer (T=32, d=256,
64 experts, top-4, f=128, int8 block-32 weights) in both activation modes, so
that any later change to the oracle's arithmetic shows up as a failing test
and has to be justified when the fixture is rewritten.

    python tests/golden/make_oracle_regression.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_layer.txt")
TOKENS = (0, 7, 19, 31)


def main():
    L = synth.make_layer("tiny", seed=0)
    c = L.cfg
    lines = ["# oracle output on the seeded tiny layer (seed 0); written by make_oracle_regression.py",
             "# ids and gates for all tokens; out rows for tokens %s; float32 as hex bit patterns" % (TOKENS,)]
    for mode, tag in ((oracle.ACT_FLOAT, "float"), (oracle.ACT_Q8, "q8")):
        o = oracle.moe_layer(L.x_f32(), L.Wr, L.bias, L.experts, L.shared, c.wfmt, c.f, c.k, act_mode=mode,
                             tokens=np.array(TOKENS, dtype=np.int32))
        if tag == "float":
            lines.append("ids " + " ".join(str(int(v)) for v in o["ids"].ravel()))
            lines.append("gates " + " ".join("%08x" % v for v in o["gates"].ravel().view(np.uint32)))
        for i, t in enumerate(TOKENS):
            lines.append("out_%s_%d " % (tag, t) + " ".join("%08x" % v for v in o["out"][i].view(np.uint32)))
    with open(OUT, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
