"""Write tests/golden/c1_oracle.json: the fp64 oracle's result on the tiny fp32 workload.

The pages print no worked numerical example, so this fixture is not a value from
the pages: it freezes the oracle's own output (computed here by ``oracle/`` only,
on the seeded inputs from ``test_weight_layers_amd.synth``) so that any later
change to the oracle or to the input recipe shows up as a failing test and has
to be justified.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from test_weight_layers_amd.configs import CONFIGS  # noqa: E402
from test_weight_layers_amd.synth import as_f64, make_inputs  # noqa: E402

SAMPLES = 16


def summary(name, x):
    x = np.asarray(x, np.float64)
    flat = x.reshape(-1)
    idx = np.linspace(0, flat.size - 1, SAMPLES).astype(np.int64)
    return {"name": name, "shape": list(x.shape), "fro": float(np.linalg.norm(flat)),
            "idx": idx.tolist(), "val": [float(flat[i]) for i in idx]}


def compute():
    cfg = CONFIGS["c1"]
    inp = make_inputs(cfg)
    w = [as_f64(t) for t in (inp.w1, inp.w3, inp.w2)]
    o, w_hat, g, ns = oracle.layer(*w, as_f64(inp.k), as_f64(inp.v), as_f64(inp.eta),
                                   as_f64(inp.q), cfg.lr, cfg.steps)
    out = []
    for tag, trip in (("G", g), ("NS", ns), ("W", w_hat)):
        for j, x in zip(("1", "3", "2"), trip):
            out.append(summary(tag + j, x))
    out.append(summary("O", o))
    return out


if __name__ == "__main__":
    data = {"workload": "c1-tiny-f32", "oracle": "fp64", "tensors": compute()}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle.json"), "w") as f:
        json.dump(data, f, indent=1)
    print("wrote c1_oracle.json")
