"""Test-side models of the attention kernels' rounding points, for tight parity checks.

These are NOT the oracle.  The oracle (``oracle/``) is the exact definition in
fp64; checked against it, the kernels' outputs carry the error of every
rounding the fast path performs (q and K to bf16 or e4m3, p to bf16 or e4m3,
the output to bf16), which at sharp softmaxes approaches the workload
tolerance and so could hide a small arithmetic bug.  The models below take the
oracle's exact rotated queries and apply the same roundings the kernels apply,
at the same points, with the keys and values read back from the cache as
stored; what remains between a kernel and its model is fp32 accumulation
order and rounding decisions taken at near-ties, so the comparison can be
held to about one bf16 ulp plus an allowance for those near-ties.

Rounding points modelled (the kernels' documented arithmetic):
* bf16 kernel: q_rot * (scale * log2 e) in fp32, rounded to bf16; scores in
  log2 units against the stored bf16 keys; p = 2^(s - m) rounded to bf16 with
  an integer running max m -- so p's bf16 significand is that of 2^s, and any
  integer shift per row gives the same normalised output; o = sum p v / sum p.
* e4m3 kernel: q_rot * (scale * log2 e * k_scale) in fp32, one power-of-two
  scale 2^e per row (the smallest e with max|x| 2^-e <= 448), codes
  e4m3(x 2^-e); scores 2^e sum q8 k8; each row walks its key split's 64-key
  tiles (cut per frame) in order, raising an integer running max m to
  ceil(tile max) when the tile max exceeds m + 8, and rounds p = 2^(s - m) to
  e4m3 (subnormals included); splits merge with weights 2^(m_s - max m_s);
  o = v_scale sum p v8 / sum p.

Near-ties.  The kernels form a score in fp32 on the matrix cores (the
products are exact; the sums round), and rotate the queries in fp32; the
models use the exact values.  Where the exact p = 2^(s - m) lies within the
score's fp32 error of a rounding midpoint of p's format, or an exact scaled
query element within the rotation's fp32 error of a midpoint of the query
format, the kernel may round to either neighbour; at e4m3 precision one such
flip on a dominant key moves the row by about a percent.  The models flag
those keys and query elements and return, per output element, the largest
change a flip can make plus a four-sigma random-sign sum of the rest
(``extra``), which the comparison adds to its allowance.  Score error bound
used: |ds| <= 2^-16 (sum_d |q_d k_d| + |m|) in log2 units.  The products are
exact and about forty fp32 roundings of partial sums no larger than that
magnitude would give 2^-18; the e4m3 matrix-core path was seen to exceed that
by up to 2x (near-midpoint keys that flipped at 1.6 - 2.0 times the 2^-18
figure), so the bound keeps a factor of four.  p's relative error is then at
most ln 2 |ds| + 2^-21 (exp2).  Rotation error bound:
2^-21 of the rotated pair's norm, times the query scale.
"""
from __future__ import annotations

import numpy as np

from oracle import fp8 as ofp8

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453
SCORE_ERR = 2.0 ** -16   # fp32 score error per unit of sum |q_d k_d| + |m| (log2 units)
EXP2_ERR = 2.0 ** -21    # relative error of the hardware exp2 on top of the score's
ROT_ERR = 2.0 ** -21     # fp32 rotation error per unit of the rotated pair's norm
FLIP_SIGMAS = 4.0        # random-sign sum of the non-dominant flips, in sigmas


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """fp64 -> fp32 -> bf16 (round to nearest even), as float64."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def scale_log2(scale: float, head_dim: int) -> float:
    """The kernels' fp32 softmax scale * log2(e) (scale 0 means 1/sqrt(D))."""
    sc = np.float32(1.0) / np.sqrt(np.float32(head_dim)) if scale == 0.0 else np.float32(scale)
    return float(np.float32(np.float64(sc) * LOG2E))


def _spacing(a, mant_bits, min_exp):
    """Spacing of a binary format with mant_bits stored mantissa bits at |a| (subnormals below 2^min_exp)."""
    _, ex = np.frexp(np.maximum(np.abs(a), 1e-300))
    return np.exp2(np.maximum(ex - 1, min_exp) - mant_bits)


def ulp_bf16(x):
    """Spacing of bf16 values at |x| (8 significant bits; normal range)."""
    return _spacing(x, 7, -126)


def ulp_e4m3(x):
    return _spacing(x, 3, -6)


def _near_midpoint(a, spacing, tol):
    """|a| lies within tol (absolute) of a rounding midpoint of a grid with the given spacing."""
    a = np.abs(a)
    mid = (np.floor(a / spacing) + 0.5) * spacing
    return np.abs(a - mid) <= tol


def _pair_norm(q):
    """Norm of each element's rotation pair (channels 2i, 2i+1), per element."""
    n = np.sqrt(q[..., 0::2] ** 2 + q[..., 1::2] ** 2)
    return np.repeat(n, 2, axis=-1)


def _flip_extra(p_amb_ulp, V_abs, o_abs, L):
    """Per-element allowance from keys whose p may round either way.

    p_amb_ulp: dict row -> (key indices, p spacing at those keys); V_abs [Lk, D] |v|; o_abs [R, D]; L [R] the
    row's normaliser.  One flip of key j changes o by at most spacing_j (|v_j| + |o|) / L."""
    R, D = o_abs.shape
    extra = np.zeros((R, D))
    for r, (idx, sp) in p_amb_ulp.items():
        if idx.size == 0:
            continue
        c = sp[:, None] * (V_abs[idx] + o_abs[r][None, :]) / L[r]   # [n_amb, D]
        extra[r] = c.max(axis=0) + FLIP_SIGMAS * np.sqrt(np.square(c).sum(axis=0))
    return extra


def _qflip_extra(amb, dq, K_abs, P, V_abs, o_abs, L):
    """Per-element allowance from query elements that may round either way.

    amb [R, D] flagged elements, dq [R, D] their spacing (score units per unit key); a flip of element d moves
    score j by dq_d |k_jd|, p_j by a factor of at most 2^(that) - 1, and o by the p-weighted sum of those."""
    R, D = amb.shape
    extra = np.zeros((R, D))
    for r in np.nonzero(amb.any(axis=1))[0]:
        ds = (K_abs[:, amb[r]] * dq[r, amb[r]][None, :]).sum(axis=1)          # worst combined score change per key
        w = P[r] * (np.exp2(ds) - 1.0) / L[r]
        extra[r] = w @ (V_abs + o_abs[r][None, :])
    return extra


def bf16_attention(q_rot, K, V, visible, sl2):
    """One head of the bf16 kernel's arithmetic.

    q_rot [Lq, D] exact rotated queries, K [Lk, D] stored keys, V [Lk, D] values, visible [Lq, Lk].  Returns
    (o [Lq, D] unrounded, extra [Lq, D] near-tie allowance)."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    x = f32(q_rot * sl2)
    qb = bf16(x)
    s = qb @ K.T
    s = np.where(visible, s, -np.inf)
    m = np.ceil(s.max(axis=1, keepdims=True))
    praw = np.exp2(s - m)
    p = np.where(visible, bf16(praw), 0.0)
    L = p.sum(axis=1)
    o = (p @ V) / L[:, None]
    # near-ties of p
    mag = np.abs(qb) @ np.abs(K).T + np.abs(m)
    tol = (LN2 * SCORE_ERR * mag + EXP2_ERR) * praw
    amb = visible & _near_midpoint(praw, ulp_bf16(praw), tol)
    p_amb = {r: (np.nonzero(amb[r])[0], ulp_bf16(praw[r, amb[r]])) for r in range(s.shape[0])}
    V_abs, o_abs = np.abs(V), np.abs(o)
    extra = _flip_extra(p_amb, V_abs, o_abs, L)
    # near-ties of the query's bf16 rounding
    qamb = _near_midpoint(x, ulp_bf16(x), ROT_ERR * _pair_norm(q_rot) * abs(sl2))
    extra += _qflip_extra(qamb, ulp_bf16(x), np.abs(K), p, V_abs, o_abs, L)
    return o, extra


def q_e4m3(q_rot, qmul):
    """The e4m3 kernel's query codes: x = fp32(q_rot * qmul), per-row e, codes e4m3(x 2^-e).

    Returns (q8 values [Lq, D], e [Lq], x [Lq, D])."""
    x = f32(np.asarray(q_rot, dtype=np.float64) * qmul)
    amax = np.abs(x).max(axis=1)
    e = np.zeros(amax.shape, dtype=np.int64)
    pos = amax > 0
    e[pos] = np.ceil(np.log2(amax[pos] / 448.0)).astype(np.int64)
    e[pos & (amax * np.exp2(-e.astype(np.float64)) > 448.0)] += 1
    e = np.clip(e, -126, 126)
    q8 = ofp8.round_e4m3(x * np.exp2(-e.astype(np.float64))[:, None])
    return q8, e, x


def e4m3_attention(q_rot, K8, V8, T, fend_row, fend_wg, n_splits, qmul, v_scale):
    """One head of the e4m3 kernel's arithmetic.

    q_rot [Lq, D] exact rotated queries; K8, V8 [n_res*T, D] decoded stored codes (k / k_scale, v / v_scale
    rounded), keys in logical order, T per frame; row r sees frames [0, fend_row[r]) and its workgroup
    walks the key tiles of frames [0, fend_wg[r]) (those its last row sees), split into n_splits
    contiguous tile ranges.  Returns (o [Lq, D] unrounded, extra [Lq, D] near-tie allowance).
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    K8 = np.asarray(K8, dtype=np.float64)
    V8 = np.asarray(V8, dtype=np.float64)
    q8, e, x = q_e4m3(q_rot, qmul)
    scale_e = np.exp2(e.astype(np.float64))
    s_all = (q8 @ K8.T) * scale_e[:, None]
    mag_all = (np.abs(q8) @ np.abs(K8).T) * scale_e[:, None]
    Lq, D = q8.shape
    ntf = (T + 63) // 64
    out = np.empty((Lq, D))
    extra = np.zeros((Lq, D))
    V_abs = np.abs(V8) * v_scale
    for wg_frames in np.unique(fend_wg):
        rows = np.nonzero(fend_wg == wg_frames)[0]
        s = s_all[rows]
        fr = fend_row[rows]
        n_tiles = int(wg_frames) * ntf
        parts = []
        for sp in range(n_splits):
            lo, hi = (n_tiles * sp) // n_splits, (n_tiles * (sp + 1)) // n_splits
            m = np.full(rows.size, -np.inf)
            O = np.zeros((rows.size, D))
            l = np.zeros(rows.size)
            keys_sp, P_sp, amb_sp, ulp_sp, mrow_sp = [], [], [], [], []
            for kt in range(lo, hi):
                lf, jl0 = kt // ntf, (kt % ntf) * 64
                keys = np.arange(lf * T + jl0, lf * T + min(jl0 + 64, T))
                vis = (lf < fr)[:, None]
                st = np.where(vis, s[:, keys], -np.inf)
                mx = st.max(axis=1)
                raise_ = mx > m + 8.0                      # per row; never for a tile it does not see
                m_new = np.where(raise_, np.ceil(np.where(raise_, mx, 0.0)), m)
                alpha = np.where(raise_ & np.isfinite(m), np.exp2(np.where(np.isfinite(m), m, 0.0) - m_new), 1.0)
                O *= alpha[:, None]
                l *= alpha
                for t in range(len(P_sp)):                  # earlier tiles of this split, re-based with m
                    P_sp[t] = P_sp[t] * alpha[:, None]
                    ulp_sp[t] = ulp_sp[t] * alpha[:, None]
                m = m_new
                m0 = np.where(np.isneginf(m), 0.0, m)
                praw = np.exp2(st - m0[:, None])
                p = np.where(vis, ofp8.round_e4m3(praw), 0.0)
                O += p @ V8[keys]
                l += p.sum(axis=1)
                tol = (LN2 * SCORE_ERR * (mag_all[rows][:, keys] + np.abs(m0)[:, None]) + EXP2_ERR) * praw
                keys_sp.append(keys)
                P_sp.append(p)
                amb_sp.append(vis & _near_midpoint(praw, ulp_e4m3(praw), tol))
                ulp_sp.append(ulp_e4m3(praw))
            parts.append((m, O * v_scale, l, keys_sp, P_sp, amb_sp, ulp_sp))
        M = np.max([pm for pm, *_ in parts], axis=0)
        num = np.zeros((rows.size, D))
        den = np.zeros(rows.size)
        ws = []
        for pm, pO, pl, *_ in parts:
            w = np.where(np.isneginf(pm), 0.0, np.exp2(np.where(np.isneginf(pm), 0.0, pm - M)))
            ws.append(w)
            num += w[:, None] * pO
            den += w * pl
        o = num / den[:, None]
        out[rows] = o
        # near-tie allowances: p flips in every split (each p weighted by its split's merge weight), then q flips
        o_abs = np.abs(o)
        keys_all = np.concatenate([k for part in parts for k in part[3]]) if parts[0][3] else np.zeros(0, int)
        if keys_all.size:
            P_w = np.concatenate([w[:, None] * P for w, part in zip(ws, parts) for P in part[4]], axis=1)
            amb_w = np.concatenate([A for part in parts for A in part[5]], axis=1)
            ulp_w = np.concatenate([w[:, None] * U for w, part in zip(ws, parts) for U in part[6]], axis=1)
            p_amb = {i: (keys_all[amb_w[i]], ulp_w[i, amb_w[i]]) for i in range(rows.size)}
            ex = _flip_extra(p_amb, V_abs, o_abs, den)
            xr = x[rows] * np.exp2(-e[rows].astype(np.float64))[:, None]
            tolq = ROT_ERR * _pair_norm(q_rot[rows]) * abs(qmul) * np.exp2(-e[rows].astype(np.float64))[:, None]
            qamb = _near_midpoint(xr, ulp_e4m3(xr), tolq)
            dq = ulp_e4m3(xr) * scale_e[rows][:, None]
            P_full = np.zeros((rows.size, K8.shape[0]))
            np.add.at(P_full.T, keys_all, P_w.T)
            ex += _qflip_extra(qamb, dq, np.abs(K8), P_full, V_abs, o_abs, den)
            extra[rows] = ex
    return out, extra


MODEL_REL = 1e-3   # rel-L2 of (kernel - bf16(model)), after the near-tie allowance: fp32 order only
MODEL_ULPS = 2.0   # per element: two bf16 ulps of the model value (its own rounding and the kernel's) ...
MODEL_FLOOR = 2.0 ** -9  # ... plus this fraction of the row's RMS (cancellation in small elements)


def model_mismatch(got, model, extra=None):
    """(rel-L2 of got - bf16(model) beyond the near-tie allowance, worst per-element excess over the
    allowance, fraction bit-equal).

    got, model, extra: [..., D] with D the last axis (rows of one head each)."""
    got = np.asarray(got, dtype=np.float64)
    model = np.asarray(model, dtype=np.float64)
    extra = np.zeros_like(model) if extra is None else np.asarray(extra, dtype=np.float64)
    mb = bf16(model)
    d = got - mb
    d_unexplained = np.sign(d) * np.maximum(np.abs(d) - extra, 0.0)
    rel = float(np.linalg.norm(d_unexplained) / max(np.linalg.norm(mb), 1e-300))
    row_rms = np.sqrt(np.mean(model ** 2, axis=-1, keepdims=True))
    allow = MODEL_ULPS * ulp_bf16(model) + MODEL_FLOOR * row_rms + extra
    excess = float(np.max(np.abs(got - model) - allow)) if got.size else -1.0
    return rel, excess, float(np.mean(d == 0.0))


def assert_matches_model(got, model, what, extra=None):
    rel, excess, eq = model_mismatch(got, model, extra)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert rel <= MODEL_REL and excess <= 0.0, \
        f"{what}: vs rounding model rel_l2 {rel:.3e} (tol {MODEL_REL}), worst element over its allowance by {excess:.3e}"
    return rel, eq
