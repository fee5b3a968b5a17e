"""Shared test helpers: run the HIP library and the oracle on the same seeded inputs."""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import torch

import oracle
from test_weight_layers_amd import synth
from test_weight_layers_amd.configs import CONFIGS, LayerConfig

TOL = {"f32": 1e-4, "bf16": 2e-2}


def cfg_like(base: str, **kw) -> LayerConfig:
    return replace(CONFIGS[base], **kw)


def conv_geometry(cfg: LayerConfig, n_tokens: int):
    frames = n_tokens // cfg.tokens_per_frame
    return dict(frames=frames, tokens_per_frame=cfg.tokens_per_frame, n_special=cfg.n_special,
                grid_h=cfg.grid_h, grid_w=cfg.grid_w)


def oracle_layer(inp: synth.LayerInputs, steps=None, lr=None, conv=None):
    """fp64 oracle on the (already rounded) inputs. Returns dict of numpy arrays."""
    cfg = inp.cfg
    steps = cfg.steps if steps is None else steps
    lr = cfg.lr if lr is None else lr
    conv_args = None
    if conv if conv is not None else cfg.conv:
        conv_args = dict(wconv=synth.as_f64(inp.wconv), **conv_geometry(cfg, inp.k.shape[0]))
    w = [synth.as_f64(t) for t in (inp.w1, inp.w3, inp.w2)]
    o, w_hat, g, ns = oracle.layer(*w, synth.as_f64(inp.k), synth.as_f64(inp.v), synth.as_f64(inp.eta),
                                   synth.as_f64(inp.q), lr, steps, conv=conv_args)
    return {"O": o, "W": w_hat, "G": g, "NS": ns}


def gpu_layer(inp: synth.LayerInputs, steps=None, lr=None, conv=None):
    """The HIP library on the same inputs (moved to cuda:0). Returns dict of numpy arrays."""
    from test_weight_layers_amd import ttt
    cfg = inp.cfg
    steps = cfg.steps if steps is None else steps
    lr = cfg.lr if lr is None else lr
    d_inp = synth.to_device(inp, "cuda")
    H, d, m = cfg.heads, cfg.d, cfg.m
    w = (d_inp.w1, d_inp.w3, d_inp.w2)
    v = d_inp.v
    if conv if conv is not None else cfg.conv:
        geo = conv_geometry(cfg, inp.k.shape[0])
        v = ttt.shortconv2d(v, d_inp.wconv, **geo)
    g = torch.empty(3 * H * m * d, dtype=torch.float32, device="cuda")
    ns = torch.empty_like(g)
    w_hat = ttt.update(w, d_inp.k, v, d_inp.eta, lr, steps, grad_out=g, ns_out=ns)
    o = ttt.apply(w_hat, d_inp.q)
    torch.cuda.synchronize()
    split = lambda t: (t[:H * m * d].view(H, m, d), t[H * m * d:2 * H * m * d].view(H, m, d),
                       t[2 * H * m * d:].view(H, d, m))
    to = lambda t: t.detach().double().cpu().numpy()
    return {"O": to(o), "W": tuple(map(to, w_hat)), "G": tuple(map(to, split(g))), "NS": tuple(map(to, split(ns)))}


def rel(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def parity_report(got, ref, heads, d):
    """Relative Frobenius error per head and matrix for G, NS(G), W^ and O."""
    rep = {}
    for key in ("G", "NS", "W"):
        for j, name in enumerate(("1", "3", "2")):
            for h in range(heads):
                rep[f"{key}{name}[h{h}]"] = rel(got[key][j][h], ref[key][j][h])
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        rep[f"O[h{h}]"] = rel(got["O"][:, c], ref["O"][:, c])
    return rep
