"""Oracle: LoL per-head jittered bases and 3D rotary position embedding (fp64).

Test infrastructure only (see ``oracle/__init__``).

Sources:
* LoL paper review, background "Rotary Position Embedding (RoPE)": a
  position t rotates channel pair i by the 2x2 matrix
  [[cos(t w_i), -sin(t w_i)], [sin(t w_i), cos(t w_i)]] with base frequency
  w_i = theta^(-2i/d), so that scores depend only on the position offset.
* LoL paper review, "method steps": (2) frequency exponents -2i/d_time;
  (3) eps_h ~ U[-1, 1] per head; (4) theta_hat_h = theta0 (1 + sigma eps_h);
  (5) w_h = theta_hat_h ** exponents; (6) rotate Q_h, K_h with w_h;
  (7) concatenate heads.

Readings taken where the pages are silent or garbled:
* The matrix row break is lost on the page; the rotation is the standard
  counter-clockwise one, R(phi) = [[cos, -sin], [sin, cos]] acting on the
  column (x_{2p}, x_{2p+1}).
* Channel pairs are adjacent, (2p, 2p+1); the head dimension is split into
  consecutive [t | h | w] segments of d_t, d_h, d_w channels.
* Frequencies use the axis' own sub-dimension: w_{a,j} = theta_a^(-2j/d_a),
  j = 0 .. d_a/2 - 1 (the page names d_time as the denominator).
* The jitter applies to the time axis by default; ``jitter_axes`` selects
  others.  One eps per head, shared by Q and K, all frames and all streams.
* Positions: t is the latent frame's time index; token i of a frame sits at
  row i // grid_w, column i % grid_w.
* Position interpolation (PI), the baseline the LoL review's results compare
  against (it compresses positions, which ends the collapse but also most of
  the motion): the time position of a frame becomes t * t_scale with a
  compression factor t_scale (1 = none); the grid positions are unchanged.
  The review gives no factor, so it is a parameter.
"""
from __future__ import annotations

import numpy as np

AXES = ("t", "h", "w")


def theta_hat(theta0: float, sigma: float, eps, jitter_axes=("t",)) -> np.ndarray:
    """Per-head, per-axis bases [H, 3]: theta0 (1 + sigma eps_h) on jittered axes, theta0 elsewhere.

    LoL paper review, method steps (3)-(4).
    """
    eps = np.asarray(eps, dtype=np.float64)
    H = eps.shape[0]
    out = np.full((H, 3), float(theta0), dtype=np.float64)
    for a, name in enumerate(AXES):
        if name in jitter_axes:
            out[:, a] = float(theta0) * (1.0 + float(sigma) * eps)
    return out


def axis_frequencies(base: float, d_axis: int) -> np.ndarray:
    """w_j = base ** (-2 j / d_axis) for j = 0 .. d_axis/2 - 1 (LoL review, background RoPE; steps 2, 5)."""
    j = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / float(d_axis))


def head_frequencies(bases_h: np.ndarray, dims) -> np.ndarray:
    """Frequencies of one head for all D/2 channel pairs, segments ordered [t | h | w]."""
    return np.concatenate([axis_frequencies(bases_h[a], dims[a]) for a in range(3)])


def pair_positions(t: int, token: np.ndarray, grid_w: int, dims, t_scale: float = 1.0) -> np.ndarray:
    """Position of every channel pair for the given tokens: [n_tokens, D/2] float64.

    The time axis sits at t * t_scale (position interpolation; 1 = none).
    """
    token = np.asarray(token, dtype=np.int64)
    pos_axes = [np.full(token.shape, float(t) * float(t_scale)), (token // grid_w).astype(np.float64),
                (token % grid_w).astype(np.float64)]
    cols = [np.repeat(pos_axes[a][:, None], dims[a] // 2, axis=1) for a in range(3)]
    return np.concatenate(cols, axis=1)


def rotate_pairs(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Apply R(phi) = [[cos, -sin], [sin, cos]] to adjacent channel pairs.

    x: [..., D]; phi broadcastable to [..., D/2].
    """
    x = np.asarray(x, dtype=np.float64)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    c = np.cos(phi)
    s = np.sin(phi)
    out = np.empty(np.broadcast_shapes(x.shape, x.shape), dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rope3d_frame(x: np.ndarray, t: int, bases: np.ndarray, dims, grid_w: int, t_scale: float = 1.0) -> np.ndarray:
    """Rotate one latent frame x [B, T_f, H, D] at time t (position t * t_scale); bases [H, 3].

    LoL review, method steps (5)-(7): each head uses its own frequencies.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, H, D = x.shape
    assert sum(dims) == D and all(d % 2 == 0 for d in dims)
    pos = pair_positions(t, np.arange(T), grid_w, dims, t_scale)  # [T, D/2]
    out = np.empty_like(x)
    for h in range(H):
        w = head_frequencies(bases[h], dims)                       # [D/2]
        out[:, :, h, :] = rotate_pairs(x[:, :, h, :], pos[None, :, :] * w[None, None, :])
    return out


def rope3d(x: np.ndarray, t0: int, tokens_per_frame: int, bases: np.ndarray, dims,
           grid_w: int, t_list=None, t_scale: float = 1.0) -> np.ndarray:
    """Rotate x [B, n*T_f, H, D]; frame j of the token axis has time t0 + j (or t_list[j])."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[1] // tokens_per_frame
    out = np.empty_like(x)
    for j in range(n):
        t = (t0 + j) if t_list is None else t_list[j]
        sl = slice(j * tokens_per_frame, (j + 1) * tokens_per_frame)
        out[:, sl] = rope3d_frame(x[:, sl], t, bases, dims, grid_w, t_scale)
    return out
