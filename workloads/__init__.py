"""Seeded synthetic inputs shared by the oracle-side and the HIP-side tests.

This module holds workload shapes and random draws only: it performs none
of the method's arithmetic (no RoPE, no attention, no projection).  Both
the oracle (fp64 numpy) and the HIP path consume exactly the tensors
produced here, so the two sides never disagree about their inputs.

Shapes follow the LongLive paper review (section 6 "implementation
details" table: Wan 2.1 1.3B base, 832x480, attention window of 12 latent
frames = 9 local + 3 sink) and the LoL paper review ("reproducibility"
paragraph: 3 sink frames, theta0 = 10000, jitter scale 0.8; "method
steps" (3): eps_h drawn from U[-1, 1] per head).  The token grid per
latent frame (30 x 52), head count (12) and head size (128) are the
Wan-1.3B token shapes of an 832x480 latent.

Seeds: numpy ``SeedSequence([base, cfg, layer, stream, frame, tensor])``.
bf16 inputs are drawn in float32 and rounded once to bfloat16
(round-to-nearest-even, torch's CPU conversion); the rounded values are
what both sides see.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_X, TENSOR_WK, TENSOR_WV, TENSOR_EPS, TENSOR_WQ, TENSOR_WO, TENSOR_XF = range(10)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int                 # 1-based config number
    batch: int               # independent streams B
    n_heads: int             # H
    head_dim: int            # D
    dims: Tuple[int, int, int]   # RoPE channels for the (t, h, w) axes
    grid: Tuple[int, int]    # (grid_h, grid_w) tokens per latent frame
    n_sink: int
    n_local: int
    chunk: int               # latent frames per append / query chunk
    frames: int              # latent frames streamed
    dtype: str               # "bf16" or "f32"
    theta0: float = 10000.0
    sigma: float = 0.0
    input_scale: float = 1.0  # Q/K/V ~ N(0,1) * input_scale
    layers: int = 1
    causal: bool = False      # frame-causal mask inside a query chunk
    hidden: int = 0           # model width C for the recache projection
    recache_after: int = -1   # recache once this many frames are streamed

    @property
    def tokens_per_frame(self) -> int:
        return self.grid[0] * self.grid[1]


WORKLOADS = {
    1: Workload("tiny-f32", 1, batch=1, n_heads=2, head_dim=64, dims=(22, 22, 20),
                grid=(8, 8), n_sink=1, n_local=2, chunk=1, frames=6, dtype="f32"),
    2: Workload("wan13b-layer-bf16", 2, batch=1, n_heads=12, head_dim=128,
                dims=(44, 42, 42), grid=(30, 52), n_sink=3, n_local=9, chunk=1,
                frames=40, dtype="bf16", input_scale=1.0 / np.sqrt(128.0)),
    3: Workload("wan13b-layer-lol-jitter", 3, batch=1, n_heads=12, head_dim=128,
                dims=(44, 42, 42), grid=(30, 52), n_sink=3, n_local=9, chunk=1,
                frames=1201, dtype="bf16", sigma=0.8, input_scale=1.0 / np.sqrt(128.0)),
    4: Workload("wan13b-prompt-switch-recache", 4, batch=1, n_heads=12, head_dim=128,
                dims=(44, 42, 42), grid=(30, 52), n_sink=3, n_local=9, chunk=1,
                frames=60, dtype="bf16", input_scale=1.0 / np.sqrt(128.0),
                hidden=1536, recache_after=30),
    5: Workload("wan13b-chunk3-b4-30layers", 5, batch=4, n_heads=12, head_dim=128,
                dims=(44, 42, 42), grid=(30, 52), n_sink=3, n_local=9, chunk=3,
                frames=30, dtype="bf16", sigma=0.8, input_scale=1.0 / np.sqrt(128.0),
                layers=30, causal=True),
}


def rng_for(cfg: int, layer: int, stream: int, frame: int, tensor: int,
            base: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([base, cfg, layer, stream, frame, tensor]))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return them as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal(shape, cfg: int, layer: int, stream: int, frame: int, tensor: int,
           scale: float = 1.0, dtype: str = "f32", base: int = 0) -> np.ndarray:
    """Seeded N(0,1)*scale draw, float32; bf16-rounded when dtype == 'bf16'."""
    g = rng_for(cfg, layer, stream, frame, tensor, base)
    x = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        x = to_bf16_values(x)
    return x


def frame_qkv(w: Workload, frame: int, layer: int = 0, tensor: int = TENSOR_Q,
              base: int = 0, scale: float | None = None) -> np.ndarray:
    """One latent frame of Q, K or V for all streams: [B, T_f, H, D] float32."""
    shape = (w.batch, w.tokens_per_frame, w.n_heads, w.head_dim)
    out = np.empty(shape, dtype=np.float32)
    s = w.input_scale if scale is None else scale
    for b in range(w.batch):
        out[b] = normal(shape[1:], w.cfg, layer, b, frame, tensor, s, w.dtype, base)
    return out


def chunk_qkv(w: Workload, first_frame: int, n_frames: int, layer: int = 0,
              tensor: int = TENSOR_Q, base: int = 0, scale: float | None = None) -> np.ndarray:
    """Frames first_frame .. first_frame+n_frames-1 concatenated on the token axis."""
    parts = [frame_qkv(w, first_frame + i, layer, tensor, base, scale) for i in range(n_frames)]
    return np.concatenate(parts, axis=1)


def head_jitter(w: Workload, layer: int = 0, base: int = 0) -> np.ndarray:
    """eps_h ~ U[-1, 1], one draw per (layer, head), fixed for the whole stream."""
    g = rng_for(w.cfg, layer, 0, 0, TENSOR_EPS, base)
    return g.uniform(-1.0, 1.0, size=w.n_heads)


def recache_inputs(w: Workload, layer: int = 0, n_frames: int | None = None, base: int = 0):
    """Hidden states x [B, n*T_f, C] ~ N(0,1) and weights W_k, W_v [C, H*D] ~ N(0, 1/C).

    Returned in the mathematical orientation K = x . W_k (W is C x H*D).
    """
    n = (w.n_sink + w.n_local) if n_frames is None else n_frames
    C = w.hidden
    HD = w.n_heads * w.head_dim
    x = np.empty((w.batch, n * w.tokens_per_frame, C), dtype=np.float32)
    for b in range(w.batch):
        x[b] = normal((n * w.tokens_per_frame, C), w.cfg, layer, b, 0, TENSOR_X, 1.0, w.dtype, base)
    wk = normal((C, HD), w.cfg, layer, 0, 0, TENSOR_WK, 1.0 / np.sqrt(C), w.dtype, base)
    wv = normal((C, HD), w.cfg, layer, 0, 0, TENSOR_WV, 1.0 / np.sqrt(C), w.dtype, base)
    return x, wk, wv


def frame_hidden(w: Workload, first_frame: int, n_frames: int = 1, layer: int = 0, base: int = 0) -> np.ndarray:
    """Hidden states of frames first_frame.. (one seed per frame and stream): [B, n*T_f, C] ~ N(0,1)."""
    T = w.tokens_per_frame
    x = np.empty((w.batch, n_frames * T, w.hidden), dtype=np.float32)
    for b in range(w.batch):
        for j in range(n_frames):
            x[b, j * T:(j + 1) * T] = normal((T, w.hidden), w.cfg, layer, b, first_frame + j, TENSOR_XF, 1.0,
                                             w.dtype, base)
    return x


def projection_weights(w: Workload, layer: int = 0, base: int = 0):
    """W_q, W_k, W_v [C, H*D] ~ N(0, 1/C) (x . W orientation), fixed per layer."""
    C, HD = w.hidden, w.n_heads * w.head_dim
    return tuple(normal((C, HD), w.cfg, layer, 0, 1, t, 1.0 / np.sqrt(C), w.dtype, base)
                 for t in (TENSOR_WQ, TENSOR_WK, TENSOR_WV))


def output_weight(w: Workload, out_features: int | None = None, layer: int = 0, base: int = 0) -> np.ndarray:
    """W_o [H*D, out] ~ N(0, 1/(H*D)) (x . W orientation); out defaults to the model width C."""
    HD = w.n_heads * w.head_dim
    out = w.hidden if out_features is None else out_features
    return normal((HD, out), w.cfg, layer, 0, 1, TENSOR_WO, 1.0 / np.sqrt(HD), w.dtype, base)
