"""The oracle against the stored record in tests/golden/oracle_tiny_layer.json
(written by tests/golden/make_golden.py, which calls only the oracle): a
change to the oracle's arithmetic must come with a regenerated record."""
import json
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_stored_record():
    rec = json.load(open(os.path.join(HERE, "oracle_tiny_layer.json")))
    s = rec["shape"]
    inp = {k: np.asarray(v, np.float32) for k, v in rec["inputs"].items()}
    y, hT, hist = oracle.mamba2_fwd(
        inp["xbc"], inp["dt"], inp["A"], nheads=s["nheads"], headdim=s["headdim"],
        ngroups=s["ngroups"], dstate=s["dstate"], conv_w=inp["conv_w"], conv_b=inp["conv_b"],
        conv_state_in=inp["conv_state_in"], D=inp["D"], dt_bias=inp["dt_bias"],
        dt_softplus=rec["dt_softplus"], z=inp["z"], h0=inp["h0"])
    exp = rec["expected"]
    np.testing.assert_allclose(y, np.asarray(exp["y"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT, np.asarray(exp["final_state"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(hist, np.asarray(exp["conv_state_out"]))
