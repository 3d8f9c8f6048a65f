"""Oracle: pure-Python loop versions for tiny shapes (pins for the numpy oracle).

Test infrastructure only (see ``oracle/__init__``).

These use only ``math`` and Python lists, with every index written out,
so they share no vectorised code path with the numpy oracle.  Same sources
and readings as ``rope``, ``attention`` and ``recache``.
"""
from __future__ import annotations

import math


def rope_vector(x, pos_per_pair, freq_per_pair):
    """Rotate one head vector x (list, length D) pair by pair."""
    out = [0.0] * len(x)
    for p in range(len(x) // 2):
        phi = pos_per_pair[p] * freq_per_pair[p]
        c, s = math.cos(phi), math.sin(phi)
        a, b = x[2 * p], x[2 * p + 1]
        out[2 * p] = a * c - b * s
        out[2 * p + 1] = a * s + b * c
    return out


def frequencies(bases_h, dims):
    """Per-pair frequency list for one head: segment a uses bases_h[a] ** (-2j/d_a)."""
    f = []
    for a in range(3):
        for j in range(dims[a] // 2):
            f.append(float(bases_h[a]) ** (-2.0 * j / dims[a]))
    return f


def positions(t, token, grid_w, dims):
    """Per-pair position list for one token: t on the time pairs, row/column on the others."""
    pos = [float(t), float(token // grid_w), float(token % grid_w)]
    out = []
    for a in range(3):
        out += [pos[a]] * (dims[a] // 2)
    return out


def attention_row(q, keys, values, scale):
    """One query against a list of keys/values with a plain two-pass softmax."""
    scores = []
    for k in keys:
        acc = 0.0
        for d in range(len(q)):
            acc += q[d] * k[d]
        scores.append(acc * scale)
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = sum(w)
    out = [0.0] * len(values[0])
    for j, v in enumerate(values):
        for d in range(len(v)):
            out[d] += (w[j] / z) * v[d]
    return out


def matvec_rows(x_rows, w_cols):
    """x [L][C] times w [C][N] with explicit triple loop."""
    L, C, N = len(x_rows), len(w_cols), len(w_cols[0])
    out = [[0.0] * N for _ in range(L)]
    for i in range(L):
        for n in range(N):
            acc = 0.0
            for c in range(C):
                acc += x_rows[i][c] * w_cols[c][n]
            out[i][n] = acc
    return out


def stream_attention(q_frames, k_frames, v_frames, times, n_sink, n_local, bases, dims, grid_w,
                     causal_chunks=None, scale=None):
    """Full brute-force stream for one stream and one head group.

    q_frames/k_frames/v_frames: list over frames f of [T_f][H][D] nested lists
    (un-rotated).  Frames are appended one chunk at a time (chunk sizes from
    ``causal_chunks``, default 1); after each append the chunk's queries attend
    over the resident frames (frame-causal inside the chunk).  Returns a list
    over frames of [T_f][H][D] outputs.
    """
    n = len(q_frames)
    chunks = causal_chunks or [1] * n
    T = len(q_frames[0])
    H = len(q_frames[0][0])
    D = len(q_frames[0][0][0])
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    outputs = [None] * n
    f0 = 0
    for c in chunks:
        last = f0 + c  # frames 0..last-1 appended
        sinks = list(range(min(n_sink, last)))
        local = list(range(max(n_sink, last - n_local), last))
        resident = sinks + local
        for fq in range(f0, last):
            frame_out = []
            for tok in range(T):
                row = []
                for h in range(H):
                    fr = frequencies(bases[h], dims)
                    qr = rope_vector(q_frames[fq][tok][h], positions(times[fq], tok, grid_w, dims), fr)
                    keys, vals = [], []
                    for fk in resident:
                        if fk > fq:
                            continue
                        for kt in range(T):
                            keys.append(rope_vector(k_frames[fk][kt][h],
                                                    positions(times[fk], kt, grid_w, dims), fr))
                            vals.append(v_frames[fk][kt][h])
                    row.append(attention_row(qr, keys, vals, scale))
                frame_out.append(row)
            outputs[fq] = frame_out
        f0 = last
    return outputs
