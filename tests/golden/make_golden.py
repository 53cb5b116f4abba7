"""Writes the stored expected values under tests/golden/ by calling only the
oracle (and the seeded input generator). Run from the repository root:

    python tests/golden/make_golden.py

The pages print no worked numeric example, so every stored value here is the
oracle's own output, kept as a regression fixture: a later change to the
oracle's arithmetic shows up as a diff of these files, and its commit must
name the passage (or the reading of it) that justifies it.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

CASES = [
    # name, shape (hc, hs, r), m, seed, extra make_inputs kwargs, config kwargs, summary only
    ("tiny_hc2_hs8_r4", (2, 8, 4), 3, 5, {"wd_std": 0.7, "wu_std": 1.5}, {}, False),
    ("tiny_hc4_hs16_r8_fullnorm", (4, 16, 8), 2, 6, {"wnorm_full": True}, {"wnorm_full": True}, False),
    ("hc4_hs2560_r320_m2", (4, 2560, 320), 2, 0, {}, {}, True),
]


def _bits(t):
    return [int(v) for v in synth.bf16_bits(t).reshape(-1)]


def main():
    for name, (hc, hs, r), m, seed, kw, ckw, summary in CASES:
        sh = synth.Shape(hc, hs, r)
        d = synth.make_inputs(m, sh, seed=seed, **kw)
        cfg = oracle.OracleConfig(hc=hc, hs=hs, r=r, **ckw)
        o = oracle.forward(cfg, d["R"], d["y"], d["inj"], d["wnorm"], d["wd"], d["wi"], d["wu"])
        rec = {"shape": {"hc": hc, "hs": hs, "r": r, "eps": cfg.eps}, "m": m, "seed": seed,
               "make_inputs": kw, "config": ckw}
        if summary:
            # real shape: inputs are regenerated from the seed; store a slice of each output
            rec["outputs"] = {"rrms": o["rrms"].tolist(), "inj_next": o["inj_next"].tolist(),
                              "x_head": o["x"][:, :16].tolist(), "R2_head": o["R2"][:, :16].tolist(),
                              "x_sum": o["x"].sum(axis=1).tolist(), "R2_sum": o["R2"].sum(axis=1).tolist()}
        else:
            rec["inputs_bf16_bits"] = {k: _bits(d[k]) for k in ("R", "y", "inj", "wnorm", "wd", "wi", "wu")}
            rec["outputs"] = {k: o[k].tolist() for k in ("R2", "rrms", "inj_next", "x")}
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(rec, f, indent=1)
        print("wrote", name)


if __name__ == "__main__":
    main()
