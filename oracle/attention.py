"""Oracle: softmax attention over the resident sink + window frames (fp64).

Test infrastructure only (see ``oracle/__init__``).

Sources:
* LongLive paper review, section 3 "Short-Window Attention": the output is
  softmax(q k_window / sqrt(d)) v_window, the window being the recent
  latent frames (plus the pinned sink frames of "Frame Sink").
* LoL paper review, background "multi-head attention": each head h
  computes softmax(Q_h K_h^T / sqrt(d_k)) V_h independently.

Readings taken:
* The scale is 1/sqrt(D) with D the head size, unless a scale is given.
* Frame-causal masking (chunk-wise generation): a query token of frame f_q
  sees every token of every resident frame f_k <= f_q; tokens of one frame
  have no order among themselves.  Without the mask a query sees all
  resident frames.
"""
from __future__ import annotations

import numpy as np


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray,
                      scale: float, return_probs: bool = False):
    """One head: q [Lq, D], k [Lk, D], v [Lk, D], visible [Lq, Lk] bool -> o [Lq, D].

    o_i = sum_j p_ij v_j with p_ij = exp(s_ij - max_j s_ij) / sum_j exp(...),
    s_ij = scale * q_i . k_j over visible j only.  Every query must see at
    least one key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    visible = np.asarray(visible, dtype=bool)
    if not visible.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = (q @ k.T) * float(scale)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(visible, np.exp(s - m), 0.0)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ v
    return (o, p) if return_probs else o


def frame_visibility(query_frames, key_frames, tokens_per_frame: int, causal: bool) -> np.ndarray:
    """Token-level visibility [Lq, Lk] from frame numbers (frame-causal or full)."""
    qf = np.repeat(np.asarray(query_frames, dtype=np.int64), tokens_per_frame)
    kf = np.repeat(np.asarray(key_frames, dtype=np.int64), tokens_per_frame)
    if not causal:
        return np.ones((qf.size, kf.size), dtype=bool)
    return kf[None, :] <= qf[:, None]


def window_attention(q_rot: np.ndarray, k_frames, v_frames, key_frames, query_frames,
                     tokens_per_frame: int, causal: bool, scale: float | None = None,
                     heads=None, rows=None) -> np.ndarray:
    """Attention of rotated queries over the resident frames.

    q_rot     : [B, n_q*T_f, H, D] rotated queries of frames ``query_frames``
    k_frames  : list of [B, T_f, H, D] rotated keys, one per resident frame
    v_frames  : list of [B, T_f, H, D] values
    key_frames: frame numbers of the resident frames (logical order)
    heads/rows: optional subsets to evaluate (large shapes are sampled)
    Returns o [B, n_rows, n_heads, D] float64.
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    B, Lq, H, D = q_rot.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    K = np.concatenate([np.asarray(k, dtype=np.float64) for k in k_frames], axis=1)
    V = np.concatenate([np.asarray(v, dtype=np.float64) for v in v_frames], axis=1)
    vis = frame_visibility(query_frames, key_frames, tokens_per_frame, causal)[rows]
    out = np.empty((B, rows.size, len(heads), D), dtype=np.float64)
    for b in range(B):
        for i, h in enumerate(heads):
            out[b, :, i, :] = softmax_attention(q_rot[b, rows, h, :], K[b, :, h, :],
                                                V[b, :, h, :], vis, scale)
    return out
