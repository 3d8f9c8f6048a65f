"""Oracle: per-frame Q/K/V projections into the cache, and a plain linear map (fp64).

Test infrastructure only (see ``oracle/__init__``).

Sources:
* LoL paper review, background "multi-head attention": each head has its
  own query, key and value projection matrices, and attention runs per head
  on the projected Q_h, K_h, V_h.
* LongLive paper review, section 3 "KV Recache": the cache is recomputed at
  a prompt switch, i.e. the key/value projections that filled it are run
  again; the per-frame projections here are the same maps applied to the
  newest frames as they are generated.

Readings taken:
* For a chunk of c new frames with hidden states x [B, c*T_f, C]:
  q = x W_q, k = x W_k, v = x W_v (W in the x . W orientation [C, H*D],
  output column h*D + d is channel d of head h, no bias).  q is returned
  un-rotated: the attention rotates its queries at their own frame time.
  (k, v) join the cache exactly as an append of those values does: K is
  rotated at each frame's time, sinks are pinned and the ring evicts.
* The pages show no output projection after the attention; ``linear`` is
  the plain x W (no bias) that a multi-head attention block closes with,
  given here because the library exports that map for it.
"""
from __future__ import annotations

import numpy as np

from . import recache as _recache


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [..., C] . w [C, F] -> [..., F] in float64."""
    return np.matmul(np.asarray(x, dtype=np.float64), np.asarray(w, dtype=np.float64))


def project_append(stream, x: np.ndarray, w_q, w_k: np.ndarray, w_v: np.ndarray, n_heads: int, t0: int):
    """Project x to (q, k, v) and append (k, v) to ``stream`` (a StreamOracle) at times t0, t0+1, ...

    Returns (q [B, c*T_f, H, D] un-rotated, or None when w_q is None; the
    frames the append evicted).
    """
    q = None if w_q is None else _recache.project(x, w_q, n_heads)
    k = _recache.project(x, w_k, n_heads)
    v = _recache.project(x, w_v, n_heads)
    evicted = stream.append(k, v, t0)
    return q, evicted
