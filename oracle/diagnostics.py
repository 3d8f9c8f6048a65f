"""Oracle: LoL's collapse diagnostics (fp64).

Test infrastructure only (see ``oracle/__init__``).

Sources:
* LoL paper review, "core method" paragraph: at a collapse several heads at
  once give the sink frames abnormally high attention weight, while normal
  frames show varied attention; "technical novelty" names this cross-head
  homogenisation.  The per-head attention weight on the sink frames is the
  quantity observed.
* LoL paper review, "core innovation" paragraph: the phase-coherence kernel
  C(Delta) = (1/K) sum_{i=1..K} exp(j w_i Delta) measures how far the RoPE
  phases line up at an offset Delta; its local maxima mark the collapses.

Readings taken:
* Sink mass of one query row in one head: the sum of that row's softmax
  probabilities (the ones the attention itself uses) over the keys of the
  resident sink frames.  A row that sees no sink key has mass 0.
* C(Delta) is taken per head over that head's time-axis frequencies
  w_{h,t,i} = base_{h,t} ** (-2i/d_t), i = 0 .. d_t/2 - 1 (K = d_t/2), Delta
  being a frame offset: the offset between a sink frame and a far frame
  changes only the time phases (a token's grid phases are the same in every
  frame), and the method builds its jittered frequencies from the time
  sub-dimension.
"""
from __future__ import annotations

import numpy as np

from . import attention as _attn
from . import rope as _rope


def sink_mass(stream, q: np.ndarray, causal: bool, scale: float | None = None, heads=None, rows=None):
    """Softmax mass on sink-frame keys for the queries q of the newest n_q frames of ``stream``.

    q: [B, n_q*T_f, H, D] un-rotated (rotated here at each query frame's time,
    as the attention does).  Returns [B, n_rows, n_heads] float64.
    """
    T = stream.T
    n_q = q.shape[1] // T
    res = stream.resident()
    qframes = res[-n_q:]
    t_list = [stream.model.t[f] for f in qframes]
    q_rot = _rope.rope3d(q, 0, T, stream.bases, stream.dims, stream.grid_w, t_list=t_list,
                         t_scale=stream.t_scale)
    B, Lq, H, D = q_rot.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    K = np.concatenate([np.asarray(stream.model.k[f], dtype=np.float64) for f in res], axis=1)
    vis = _attn.frame_visibility(qframes, res, T, causal)[rows]
    is_sink = np.repeat(np.array([f < stream.model.n_sink for f in res]), T)
    dummy_v = np.zeros((K.shape[1], 1))
    out = np.empty((B, rows.size, len(heads)), dtype=np.float64)
    for b in range(B):
        for i, h in enumerate(heads):
            _, p = _attn.softmax_attention(q_rot[b, rows, h, :], K[b, :, h, :], dummy_v, vis, scale,
                                           return_probs=True)
            out[b, :, i] = p[:, is_sink].sum(axis=1)
    return out


def phase_coherence(bases: np.ndarray, dims, deltas, t_scale: float = 1.0) -> np.ndarray:
    """C_h(Delta) for every head h (rows) and offset Delta (columns), complex128 [H, n].

    Under position interpolation a frame offset Delta is a time-position offset
    Delta * t_scale.
    """
    bases = np.asarray(bases, dtype=np.float64)
    deltas = np.asarray(deltas, dtype=np.float64) * float(t_scale)
    out = np.empty((bases.shape[0], deltas.size), dtype=np.complex128)
    for h in range(bases.shape[0]):
        w = _rope.axis_frequencies(bases[h, 0], dims[0])       # time axis
        out[h] = np.exp(1j * np.outer(deltas, w)).mean(axis=1)
    return out
