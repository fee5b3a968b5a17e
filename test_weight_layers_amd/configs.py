"""Workload shapes for the large-chunk TTT (LaCT) layer.

Token counts follow the frame layouts the pages describe:

* VGGT-style frames (VGG-T3 "方法详解 / 关键设计 2", ZipMap "整体框架"): a 518x518
  image at patch 14 gives a 37x37 patch grid plus 5 camera/register tokens,
  1374 tokens per frame.
* tttLRM object views ("方法步骤详情"): 256x256 at patch 8 gives 32x32 = 1024
  tokens per view; query-only "virtual" tokens only go through Apply.
* ZipMap ray-map queries ("关键设计 4"): target views enter as query-only tokens.
* LoGeR ("方法概览"): the stream is cut into consecutive chunks; the fast weights
  are updated from each chunk and carried to the next.

The per-head split (4 heads of 256 with SwiGLU hidden 512 for a 1024-wide
token) is a workload choice, not something the pages fix; ZipMap's own state
(d=1024, hidden 2048) is a separate shape below.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

VGGT_GRID = 37          # 518 / 14
VGGT_SPECIAL = 5        # camera + register tokens per frame
VGGT_TOKENS = VGGT_GRID * VGGT_GRID + VGGT_SPECIAL   # 1374


@dataclass(frozen=True)
class LayerConfig:
    name: str
    heads: int
    d: int                 # per-head key/value width
    m: int                 # SwiGLU hidden width per head
    frames: int            # frames (views) whose tokens form the update set
    tokens_per_frame: int
    grid_h: int            # patch grid of one frame (for ShortConv2D)
    grid_w: int
    n_special: int         # non-patch tokens at the start of each frame
    extra_query: int       # query-only tokens appended after the input tokens
    steps: int             # inner Muon steps per update
    conv: bool             # V' = ShortConv2D(V) before the update
    dtype: str             # "bf16" or "f32" token storage
    seed: int
    lr: float = 0.01
    norm_q: bool = True    # Q, K L2-normalised per token and head
    norm_k: bool = True
    norm_v: bool = False
    chunk_frames: int = 0  # >0: streaming, apply-then-update per chunk
    norm_preserve: bool = False   # ZipMap's norm-preserving weight step
    gate: bool = False     # ZipMap's gated output unit on the apply rows
    gate_eps: float = 1e-6

    @property
    def n(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def nq(self) -> int:
        return self.n + self.extra_query

    @property
    def width(self) -> int:
        return self.heads * self.d

    def with_frames(self, frames: int, extra_query: int | None = None) -> "LayerConfig":
        kw = {"frames": frames}
        if extra_query is not None:
            kw["extra_query"] = extra_query
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 layer: 4 frames x 64 tokens (an 8x8 grid, no special tokens).
    "c1": LayerConfig("c1-tiny-f32", heads=1, d=64, m=128, frames=4, tokens_per_frame=64,
                      grid_h=8, grid_w=8, n_special=0, extra_query=0, steps=1, conv=False,
                      dtype="f32", seed=0),
    # tttLRM object scale: 8 views of 1024 tokens, 8192 query-only tokens.
    "c2": LayerConfig("c2-tttlrm-object", heads=1, d=768, m=768, frames=8, tokens_per_frame=1024,
                      grid_h=32, grid_w=32, n_special=0, extra_query=8192, steps=1, conv=False,
                      dtype="bf16", seed=1, norm_v=True),
    # VGGT scale, 100 frames, ShortConv2D on V.
    "c3": LayerConfig("c3-vggt-100", heads=4, d=256, m=512, frames=100, tokens_per_frame=VGGT_TOKENS,
                      grid_h=VGGT_GRID, grid_w=VGGT_GRID, n_special=VGGT_SPECIAL, extra_query=0,
                      steps=1, conv=True, dtype="bf16", seed=2),
    # ZipMap scale, 750 frames, plus 64 query-only ray frames.
    "c4": LayerConfig("c4-zipmap-750", heads=4, d=256, m=512, frames=750, tokens_per_frame=VGGT_TOKENS,
                      grid_h=VGGT_GRID, grid_w=VGGT_GRID, n_special=VGGT_SPECIAL,
                      extra_query=64 * VGGT_TOKENS, steps=1, conv=False, dtype="bf16", seed=3),
    # VGG-T3 test-time scaling: 1000 frames, ShortConv2D, two inner steps.
    "c5a": LayerConfig("c5a-vggt3-1k", heads=4, d=256, m=512, frames=1000, tokens_per_frame=VGGT_TOKENS,
                       grid_h=VGGT_GRID, grid_w=VGGT_GRID, n_special=VGGT_SPECIAL, extra_query=0,
                       steps=2, conv=True, dtype="bf16", seed=4),
    # LoGeR-style causal stream: 4000 frames in 32-frame chunks, W carried.
    "c5b": LayerConfig("c5b-loger-stream", heads=4, d=256, m=512, frames=4000,
                       tokens_per_frame=VGGT_TOKENS, grid_h=VGGT_GRID, grid_w=VGGT_GRID,
                       n_special=VGGT_SPECIAL, extra_query=0, steps=1, conv=False, dtype="bf16",
                       seed=5, chunk_frames=32),
    # ZipMap-750 with ZipMap's stabilisers: norm-preserving step, gated output.
    "c4z": LayerConfig("c4z-zipmap-750-stabilised", heads=4, d=256, m=512, frames=750,
                       tokens_per_frame=VGGT_TOKENS, grid_h=VGGT_GRID, grid_w=VGGT_GRID,
                       n_special=VGGT_SPECIAL, extra_query=64 * VGGT_TOKENS, steps=1, conv=False,
                       dtype="bf16", seed=3, norm_preserve=True, gate=True),
    # ZipMap's own single-state shape (d=1024, hidden 2048, 6d^2 state).
    "zipmap1h": LayerConfig("zipmap-1head-d1024", heads=1, d=1024, m=2048, frames=750,
                            tokens_per_frame=VGGT_TOKENS, grid_h=VGGT_GRID, grid_w=VGGT_GRID,
                            n_special=VGGT_SPECIAL, extra_query=0, steps=1, conv=False,
                            dtype="bf16", seed=6),
}
