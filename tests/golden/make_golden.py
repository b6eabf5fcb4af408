"""Writes oracle_tiny_layer.json: a small Mamba-2 layer case (conv + SiLU over
x|B|C, selective scan with initial state, D skip, SiLU(z) gate) with its
inputs and the fp64 oracle's outputs, so that any later change to the
oracle's arithmetic shows up as a diff against this file.

The pages print no worked example of the layer, so this fixture is a
regression record of the oracle, not an independent pin; the pins are the
closed forms and brute-force forms in tests/test_oracle_pins.py.  The
recurrence it records is the one of "Hybrid Architectures for Language
Models: Systematic Analysis and Design Insights" (Korean summary), section 2
Background; the conv width 4 and SiLU come from "Nemotron-H style Hybrid
Mamba-Transformer 3B feasibility study", table 1.4.

Run from the repository root:  python tests/golden/make_golden.py
It calls only oracle/ (and numpy for the inputs).
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_layer.json")
SHAPE = dict(batch=2, seqlen=11, nheads=2, headdim=3, ngroups=1, dstate=4, width=4)


def inputs():
    s = SHAPE
    B, L, H, P, G, N, K = (s[k] for k in ("batch", "seqlen", "nheads", "headdim", "ngroups",
                                          "dstate", "width"))
    C = H * P + 2 * G * N
    rng = np.random.Generator(np.random.PCG64(20260305))
    r32 = lambda *shape, sc=1.0: (sc * rng.standard_normal(shape)).astype(np.float32)
    return dict(
        xbc=r32(B, L, C), dt=r32(B, L, H, sc=0.5), z=r32(B, L, H, P),
        conv_w=r32(C, K, sc=0.25), conv_b=r32(C, sc=0.1), conv_state_in=r32(B, K - 1, C),
        A=-np.array([1.5, 0.25], np.float32), D=np.array([1.0, -0.5], np.float32),
        dt_bias=np.array([-1.0, 0.5], np.float32), h0=r32(B, H, P, N, sc=0.1))


def run(inp):
    s = SHAPE
    return oracle.mamba2_fwd(
        inp["xbc"], inp["dt"], inp["A"], nheads=s["nheads"], headdim=s["headdim"],
        ngroups=s["ngroups"], dstate=s["dstate"], conv_w=inp["conv_w"], conv_b=inp["conv_b"],
        conv_state_in=inp["conv_state_in"], D=inp["D"], dt_bias=inp["dt_bias"],
        dt_softplus=True, z=inp["z"], h0=inp["h0"])


def main():
    oracle.build(force=False)
    inp = inputs()
    y, hT, hist = run(inp)
    rec = {"source": "fp64 oracle record (regression, not a pin): the recurrence of 'Hybrid "
                     "Architectures for Language Models: Systematic Analysis and Design Insights' "
                     "(Korean summary), section 2 Background; conv width 4 + SiLU of 'Nemotron-H "
                     "style Hybrid Mamba-Transformer 3B feasibility study', table 1.4",
           "shape": SHAPE, "dt_softplus": True,
           "inputs": {k: v.tolist() for k, v in inp.items()},
           "expected": {"y": y.tolist(), "final_state": hT.tolist(),
                        "conv_state_out": hist.tolist()}}
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=0)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
