"""Oracle: the append-then-attend stream over a sink + window cache (fp64).

Test infrastructure only (see ``oracle/__init__``).

Composes ``rope``, ``cache``, ``attention`` and ``recache`` in the order the
LongLive paper review describes generation: frame-level autoregression with a
KV cache (section 2 "solution overview"), a frame's KV joins the cache and
its queries attend over the pinned sinks plus the local window (section 3
"Short-Window Attention" / "Frame Sink"), and a prompt switch rebuilds the
cache of the resident frames (section 3 "KV Recache").
"""
from __future__ import annotations

import numpy as np

from . import attention as _attn
from . import cache as _cache
from . import recache as _recache
from . import rope as _rope


class StreamOracle:
    """Reference stream for one layer: cache contents and attention outputs in fp64."""

    def __init__(self, n_sink, n_local, tokens_per_frame, grid_w, dims, bases, t_scale=1.0):
        self.model = _cache.CacheModel(n_sink, n_local)
        self.t_scale = float(t_scale)  # time positions t * t_scale (position interpolation)
        self.T = tokens_per_frame
        self.grid_w = grid_w
        self.dims = tuple(dims)
        self.bases = np.asarray(bases, dtype=np.float64)

    def append(self, k: np.ndarray, v: np.ndarray, t0: int):
        """k, v: [B, c*T_f, H, D] un-rotated.  K is stored rotated at each frame's time."""
        c = k.shape[1] // self.T
        k_rot = _rope.rope3d(k, t0, self.T, self.bases, self.dims, self.grid_w, t_scale=self.t_scale)
        kf = [k_rot[:, j * self.T:(j + 1) * self.T] for j in range(c)]
        vf = [np.asarray(v[:, j * self.T:(j + 1) * self.T], dtype=np.float64) for j in range(c)]
        return self.model.append(c, t0, kf, vf)

    def resident(self):
        return self.model.resident()

    def frame_kv(self, frame: int):
        return self.model.k[frame], self.model.v[frame]

    def attend(self, q: np.ndarray, causal: bool, scale=None, heads=None, rows=None):
        """q: [B, n_q*T_f, H, D] un-rotated queries of the newest n_q resident frames."""
        n_q = q.shape[1] // self.T
        res = self.resident()
        qframes = res[-n_q:]
        t_list = [self.model.t[f] for f in qframes]
        q_rot = _rope.rope3d(q, 0, self.T, self.bases, self.dims, self.grid_w, t_list=t_list,
                             t_scale=self.t_scale)
        return _attn.window_attention(q_rot, [self.model.k[f] for f in res],
                                      [self.model.v[f] for f in res], res, qframes, self.T,
                                      causal, scale, heads, rows)

    def recache(self, x: np.ndarray, w_k: np.ndarray, w_v: np.ndarray):
        """x [B, n_res*T_f, C] in logical order; W in the x . W orientation [C, H*D]."""
        res = self.resident()
        H = self.model.k[res[0]].shape[2] if res else None
        t_list = [self.model.t[f] for f in res]
        kf, vf = _recache.recache(x, w_k, w_v, H, t_list, self.T, self.bases, self.dims, self.grid_w,
                                  self.t_scale)
        for f, kk, vv in zip(res, kf, vf):
            self.model.k[f] = kk
            self.model.v[f] = vv

    def reset(self):
        self.model.reset()
