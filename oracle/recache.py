"""Oracle: KV recache at a prompt switch (fp64).

Test infrastructure only (see ``oracle/__init__``).

Source: LongLive paper review, section 3 "KV Recache": at a prompt
switch the cache is rebuilt from the already generated frames paired with
the new prompt -- the cached frames' keys and values are recomputed, then
generation continues with the new cache.

Readings taken:
* The recomputation is the key/value projection of the cached frames'
  hidden states x (which already carry the new prompt's context):
  K_f = RoPE(x_f W_k, t_f), V_f = x_f W_v, for every resident frame f
  (sinks and local frames), with no bias and no normalisation.
* Output column h*D + d of x W is channel d of head h.
* The resident set, slots and time positions do not change.
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope


def project(x: np.ndarray, w: np.ndarray, n_heads: int) -> np.ndarray:
    """x [B, L, C] . w [C, H*D] -> [B, L, H, D] in float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = np.matmul(x, w)
    B, L, HD = y.shape
    return y.reshape(B, L, n_heads, HD // n_heads)


def recache(x: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, n_heads: int,
            t_list, tokens_per_frame: int, bases: np.ndarray, dims, grid_w: int, t_scale: float = 1.0):
    """Recompute the cache of the resident frames given in logical order.

    x: [B, n*T_f, C]; returns (k_frames, v_frames), lists of [B, T_f, H, D],
    keys rotated at each frame's own time t_list[j].
    """
    k = project(x, w_k, n_heads)
    v = project(x, w_v, n_heads)
    k_frames, v_frames = [], []
    for j, t in enumerate(t_list):
        sl = slice(j * tokens_per_frame, (j + 1) * tokens_per_frame)
        k_frames.append(_rope.rope3d_frame(k[:, sl], t, bases, dims, grid_w, t_scale))
        v_frames.append(v[:, sl])
    return k_frames, v_frames
