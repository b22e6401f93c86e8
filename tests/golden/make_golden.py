"""Write oracle_small.json: a small regression fixture produced by the CPU oracle only.

Run from the repository root:  python tests/golden/make_golden.py
Inputs come from the seeded generator; every stored value is computed here by `oracle/`.
The fixture guards the oracle against unintended changes; its pins are in tests/pins.py.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import oracle as O  # noqa: E402

CFG = dict(name="tiny", heads=1, head_dim=64, grid=(1, 10, 20), block=64)  # N = 200, M = 4
TOP_P = 0.6
ROWS = [0, 63, 64, 199]


def build():
    cfg = synth.workload(**CFG)
    q, k, v = synth.make_qkv(cfg)
    qd, kd, vd = (synth.to_f64(x) for x in (q, k, v))
    s = cfg.head_dim ** -0.5
    probs = O.block_scores(qd, kd, cfg.block, s)
    sel = O.topp_select(probs, TOP_P)
    out = O.masked_attention(qd, kd, vd, cfg.block, s, sel["mask"])
    return {
        "_about": "Written by tests/golden/make_golden.py from oracle/ only (regression fixture).",
        "config": {**CFG, "grid": list(CFG["grid"]), "top_p": TOP_P, "sm_scale": s},
        "probs": probs[0, 0].tolist(),
        "mask": sel["mask"][0, 0].astype(int).tolist(),
        "kept_mass": sel["mass"][0, 0].tolist(),
        "rows": ROWS,
        "out_rows": out[0, 0, ROWS].tolist(),
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
