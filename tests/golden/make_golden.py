"""Write the frozen fp64 oracle results under tests/golden/.

* ``c1_oracle.json``: the tiny fp32 workload (one step, no ShortConv2D).
* ``c3tiny_conv_oracle.json``: a tiny layer with VGG-T3's ShortConv2D on V over
  two 37x37-grid frames (5 special tokens each) and two inner steps, the branch
  of the layer that the c1 workload never takes.

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
from dataclasses import replace

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


# the tiny conv workload: the c3 layout (VGGT frames, ShortConv2D) at 1 head of 64/128,
# 2 frames, 2 inner steps, fp32 tokens
CONV_CASE = dict(base="c3", heads=1, d=64, m=128, frames=2, steps=2, dtype="f32")


def _cfg(name):
    if name == "c1":
        return CONFIGS["c1"]
    kw = dict(CONV_CASE)
    return replace(CONFIGS[kw.pop("base")], **kw)


def compute(name="c1"):
    cfg = _cfg(name)
    inp = make_inputs(cfg)
    w = [as_f64(t) for t in (inp.w1, inp.w3, inp.w2)]
    conv = None
    if cfg.conv:
        conv = dict(wconv=as_f64(inp.wconv), frames=cfg.frames, tokens_per_frame=cfg.tokens_per_frame,
                    n_special=cfg.n_special, grid_h=cfg.grid_h, grid_w=cfg.grid_w)
    o, w_hat, g, ns = oracle.layer(*w, as_f64(inp.k), as_f64(inp.v), as_f64(inp.eta),
                                   as_f64(inp.q), cfg.lr, cfg.steps, conv=conv)
    out = []
    for tag, trip in (("G", g), ("NS", ns), ("W", w_hat)):
        for j, x in zip(("1", "3", "2"), trip):
            out.append(summary(tag + j, x))
    out.append(summary("O", o))
    return out


FILES = {"c1": "c1_oracle.json", "c3tiny_conv": "c3tiny_conv_oracle.json"}

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for name, fname in FILES.items():
        data = {"workload": _cfg(name).name if name == "c1" else "c3 layout, " + json.dumps(CONV_CASE),
                "oracle": "fp64", "tensors": compute(name)}
        with open(os.path.join(here, fname), "w") as f:
            json.dump(data, f, indent=1)
        print("wrote", fname)
