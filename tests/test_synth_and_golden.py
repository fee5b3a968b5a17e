"""Input generator properties and the frozen fp64 oracle result on the tiny workload."""
import json
import os

import numpy as np
import pytest
import torch

from test_weight_layers_amd.configs import CONFIGS, VGGT_TOKENS
from test_weight_layers_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_prefix_stable_and_deterministic():
    cfg = CONFIGS["c3"]
    a = synth.token_rows(2, "k", 40000, 4, 256, True, torch.bfloat16)
    b = synth.token_rows(2, "k", 20000, 4, 256, True, torch.bfloat16)
    c = synth.token_rows(2, "k", 40000, 4, 256, True, torch.bfloat16)
    assert torch.equal(a[:20000], b) and torch.equal(a, c)
    e1 = synth.eta_rows(2, 40000, 4)
    e2 = synth.eta_rows(2, 17000, 4)
    assert torch.equal(e1[:, :17000], e2)
    assert cfg.n == 100 * VGGT_TOKENS


def test_streams_independent_and_ranges():
    k = synth.token_rows(0, "k", 1000, 2, 64, True, torch.float32)
    v = synth.token_rows(0, "v", 1000, 2, 64, False, torch.float32)
    assert not torch.equal(k, v)
    nrm = k.reshape(1000, 2, 64).norm(dim=2)
    assert torch.allclose(nrm, torch.ones_like(nrm), atol=1e-6)
    assert abs(v.std().item() - 1.0) < 0.02
    eta = synth.eta_rows(0, 5000, 3)
    assert eta.min() >= 0 and eta.max() < 0.1 and eta.shape == (3, 5000)
    w1, w3, w2 = synth.fast_weights(0, 2, 64, 128)
    assert w1.shape == (2, 128, 64) and w2.shape == (2, 64, 128)
    assert abs(w1.std().item() - 0.02) < 0.001


def test_bf16_rounding_is_nearest_even():
    x = synth.token_rows(7, "q", 3000, 1, 64, False, torch.float32)
    y = synth.token_rows(7, "q", 3000, 1, 64, False, torch.bfloat16)
    u = x.numpy().view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(rne, y.view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("name", ["c1", "c3tiny_conv"])
def test_golden_oracle_unchanged(name):
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(HERE, "golden", mg.FILES[name])) as f:
        stored = json.load(f)["tensors"]
    now = mg.compute(name)
    for s, n in zip(stored, now):
        assert s["name"] == n["name"] and s["shape"] == n["shape"]
        assert abs(s["fro"] - n["fro"]) <= 1e-12 * max(1.0, abs(s["fro"]))
        np.testing.assert_allclose(n["val"], s["val"], rtol=1e-10, atol=1e-15)
