"""The oracle reproduces its stored regression fixtures (tests/golden/*.json,
written by tests/golden/make_golden.py from the oracle alone), and the seeded
generator still draws the stored input bits."""
import glob
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


@pytest.mark.parametrize("path", GOLDEN, ids=os.path.basename)
def test_golden(path):
    rec = json.load(open(path))
    s = rec["shape"]
    sh = synth.Shape(s["hc"], s["hs"], s["r"])
    d = synth.make_inputs(rec["m"], sh, seed=rec["seed"], **rec["make_inputs"])
    if "inputs_bf16_bits" in rec:
        for k, bits in rec["inputs_bf16_bits"].items():
            assert synth.bf16_bits(d[k]).reshape(-1).tolist() == bits, k
    cfg = oracle.OracleConfig(hc=s["hc"], hs=s["hs"], r=s["r"], eps=s["eps"], **rec["config"])
    o = oracle.forward(cfg, d["R"], d["y"], d["inj"], d["wnorm"], d["wd"], d["wi"], d["wu"])
    want = rec["outputs"]
    got = dict(o)
    got["x_head"] = o["x"][:, :16]
    got["R2_head"] = o["R2"][:, :16]
    got["x_sum"] = o["x"].sum(axis=1)
    got["R2_sum"] = o["R2"].sum(axis=1)
    for k, v in want.items():
        np.testing.assert_allclose(got[k], np.array(v), rtol=1e-12, atol=1e-14, err_msg=k)
