"""Seeded synthetic inputs for the LaCT layer (shared by the tests, the bench and smoke).

This module draws numbers and lays them out; it holds none of the layer's
arithmetic.  Recipe (per workload in ``configs.py``):

* Fast weights W1, W3 in [H, m, d] and W2 in [H, d, m], fp32, N(0, 0.02).
* ShortConv2D weights [H*d, 3, 3], fp32, N(0, 0.1).
* K, V, Q token rows [rows, H*d] drawn N(0, 1) in fp32; Q and K (and V where the
  workload says so) are L2-normalised per token and per head slice, dividing by
  max(||x||, 1e-12) -- the parameter-free normalisation that replaces LayerNorm
  on Q/K (VGG-T3, 关键设计 1).  Then rounded to nearest-even into the token dtype.
* Per-token learning rates eta in [H, N], fp32, U[0, 0.1).
* Gated-output unit: input rows o' [rows, C] N(0, 1) in the token dtype; gate
  matrix W_g [C, C] N(0, 1/C) (unit-variance pre-activations) in the token dtype;
  RMSNorm scale gamma [C] fp32, U[0.5, 1.5).

Every tensor is drawn in row blocks of ``ROW_BLOCK`` tokens, block b of stream s
from ``SeedSequence(seed, spawn_key=(s, b))`` (PCG64), so any N-prefix of a
workload is bit-identical across N and blocks can be drawn in parallel threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerConfig

ROW_BLOCK = 16384
STREAMS = ("w", "conv", "k", "v", "q", "q_extra", "eta", "gate_in", "gate_w")
TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _rng(seed: int, stream: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(STREAMS.index(stream), block))
    return np.random.Generator(np.random.PCG64(ss))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _blocks(rows: int):
    return [(b, b * ROW_BLOCK, min(rows, (b + 1) * ROW_BLOCK))
            for b in range((rows + ROW_BLOCK - 1) // ROW_BLOCK)]


def token_rows(seed: int, stream: str, rows: int, heads: int, d: int, normalize: bool,
               dtype: torch.dtype, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[rows, heads*d] standard-normal token rows (optionally L2-normalised per head)."""
    if out is None:
        out = torch.empty((rows, heads * d), dtype=dtype)
    assert out.shape == (rows, heads * d) and out.dtype == dtype

    def fill(blk):
        b, r0, r1 = blk
        x = _rng(seed, stream, b).standard_normal((r1 - r0, heads * d), dtype=np.float32)
        if normalize:
            x3 = x.reshape(r1 - r0, heads, d)
            nrm = np.sqrt(np.einsum("rhd,rhd->rh", x3, x3, dtype=np.float32))
            x3 /= np.maximum(nrm, np.float32(1e-12))[:, :, None]
        out[r0:r1].copy_(torch.from_numpy(x))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, _blocks(rows)))
    return out


def eta_rows(seed: int, rows: int, heads: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[heads, rows] fp32 per-token rates, U[0, 0.1)."""
    if out is None:
        out = torch.empty((heads, rows), dtype=torch.float32)

    def fill(blk):
        b, r0, r1 = blk
        x = _rng(seed, "eta", b).random((r1 - r0, heads), dtype=np.float32) * np.float32(0.1)
        out[:, r0:r1].copy_(torch.from_numpy(np.ascontiguousarray(x.T)))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, _blocks(rows)))
    return out


def fast_weights(seed: int, heads: int, d: int, m: int):
    """(W1 [H,m,d], W3 [H,m,d], W2 [H,d,m]) fp32, N(0, 0.02), drawn in that order."""
    g = _rng(seed, "w", 0)
    w1 = g.standard_normal((heads, m, d), dtype=np.float32) * np.float32(0.02)
    w3 = g.standard_normal((heads, m, d), dtype=np.float32) * np.float32(0.02)
    w2 = g.standard_normal((heads, d, m), dtype=np.float32) * np.float32(0.02)
    return torch.from_numpy(w1), torch.from_numpy(w3), torch.from_numpy(w2)


def conv_weights(seed: int, channels: int) -> torch.Tensor:
    """[channels, 3, 3] fp32 depthwise taps, N(0, 0.1)."""
    g = _rng(seed, "conv", 0)
    return torch.from_numpy(g.standard_normal((channels, 3, 3), dtype=np.float32) * np.float32(0.1))


def gate_weights(seed: int, channels: int, dtype: torch.dtype):
    """(W_g [C, C] in `dtype`, N(0, 1/C); gamma [C] fp32, U[0.5, 1.5))."""
    g = _rng(seed, "gate_w", 0)
    wg = g.standard_normal((channels, channels), dtype=np.float32) * np.float32(channels ** -0.5)
    gamma = np.float32(0.5) + g.random(channels, dtype=np.float32)
    return torch.from_numpy(wg).to(dtype), torch.from_numpy(gamma)


def gate_rows(seed: int, rows: int, channels: int, dtype: torch.dtype) -> torch.Tensor:
    """[rows, C] N(0, 1) input rows o' of the gated-output unit."""
    return token_rows(seed, "gate_in", rows, 1, channels, False, dtype)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    wconv: Optional[torch.Tensor]
    k: torch.Tensor          # [N, H*d]
    v: torch.Tensor          # [N, H*d]
    q: torch.Tensor          # [Nq, H*d]: N input-token queries, then query-only rows
    eta: torch.Tensor        # [H, N]


def make_inputs(cfg: LayerConfig, n: Optional[int] = None, nq_extra: Optional[int] = None,
                device: Optional[str] = None) -> LayerInputs:
    """Draw one workload's inputs; ``n`` / ``nq_extra`` override the token counts."""
    n = cfg.n if n is None else n
    extra = cfg.extra_query if nq_extra is None else nq_extra
    dt = TORCH_DTYPES[cfg.dtype]
    H, d, m = cfg.heads, cfg.d, cfg.m
    w1, w3, w2 = fast_weights(cfg.seed, H, d, m)
    wconv = conv_weights(cfg.seed, H * d) if cfg.conv else None
    k = token_rows(cfg.seed, "k", n, H, d, cfg.norm_k, dt)
    v = token_rows(cfg.seed, "v", n, H, d, cfg.norm_v, dt)
    q = torch.empty((n + extra, H * d), dtype=dt)
    token_rows(cfg.seed, "q", n, H, d, cfg.norm_q, dt, out=q[:n])
    if extra:
        token_rows(cfg.seed, "q_extra", extra, H, d, cfg.norm_q, dt, out=q[n:])
    eta = eta_rows(cfg.seed, n, H)
    inp = LayerInputs(cfg, w1, w3, w2, wconv, k, v, q, eta)
    if device is not None:
        inp = to_device(inp, device)
    return inp


def to_device(inp: LayerInputs, device: str) -> LayerInputs:
    mv = lambda t: None if t is None else t.to(device, non_blocking=False).contiguous()
    return LayerInputs(inp.cfg, mv(inp.w1), mv(inp.w3), mv(inp.w2), mv(inp.wconv),
                       mv(inp.k), mv(inp.v), mv(inp.q), mv(inp.eta))


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (bf16 or fp32) CPU/GPU tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
