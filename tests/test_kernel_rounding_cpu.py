"""CPU tests of the rounding-model check (tests/kernel_rounding.py): it accepts the kernels' own
arithmetic (fp32 accumulation, fp32 exp2, the same roundings, scores off by fp32-level errors that make
near-tie roundings go either way) and rejects plausible kernel bugs -- one 64-key tile dropped, one key
split's partial weighted 5 % wrong -- by a wide margin.  For the e4m3 kernel those bugs stay inside the
rounding noise that a correct kernel shows against the exact oracle, so only the model check can tell
them apart; for bf16 it holds the kernel to about one ulp where the exact-oracle tolerance leaves
several times that.

The "kernel" here is a float32 re-computation of each model (what the GPU does, up to summation
order), with every score perturbed by random noise of the size of the matrix cores' fp32 rounding (a
standard deviation of 2^-19 of sum |q_d k_d| + 8, inside the models' 2^-16 bound); the bugs are planted
in copies of it.  Inputs have the Wan-1.3B layer's key count (12 frames of 1560 tokens) for one head and
64 query rows."""
import numpy as np
import pytest

import kernel_rounding as kr
from oracle import attention as oattn
from oracle import fp8 as ofp8

T, N_FR, D = 1560, 12, 128


def _inputs(sharp: bool, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((64, D))
    k = kr.bf16(rng.standard_normal((N_FR * T, D)))
    v = kr.bf16(rng.standard_normal((N_FR * T, D)) / np.sqrt(128.0))
    scale = 0.25 if sharp else 0.0
    return q, k, v, scale


def _score_noise(q, K, seed):
    """fp32-level score errors: N(0, 1) * 2^-19 * (sum_d |q_d k_d| + 8), float32 [rows, keys]."""
    rng = np.random.default_rng(seed)
    mag = np.abs(q).astype(np.float64) @ np.abs(K).astype(np.float64).T + 8.0
    return (rng.standard_normal(mag.shape) * 2.0 ** -19 * mag).astype(np.float32)


def _f32_bf16_kernel(q_rot, K, V, sl2, drop=None, splits=1, split_gain=None):
    """The bf16 kernel's arithmetic in float32, split into contiguous key ranges merged by max; optional
    planted bugs: a dropped key range, or one split's partial multiplied by a gain."""
    qb = kr.bf16(np.float32(q_rot) * np.float32(sl2)).astype(np.float32)
    K32, V32 = K.astype(np.float32), V.astype(np.float32)
    noise = _score_noise(qb, K32, seed=11)
    n = K.shape[0]
    parts = []
    for sp in range(splits):
        lo, hi = n * sp // splits, n * (sp + 1) // splits
        s = qb @ K32[lo:hi].T + noise[:, lo:hi]
        if drop is not None:
            a, b = drop
            s[:, max(a - lo, 0):max(min(b - lo, hi - lo), 0)] = -np.inf
        m = np.ceil(s.max(axis=1, keepdims=True))
        p = kr.bf16(np.exp2(s - m)).astype(np.float32)
        O, l = p @ V32[lo:hi], p.sum(axis=1, keepdims=True, dtype=np.float32)
        if split_gain is not None and sp == split_gain[0]:
            O = O * np.float32(split_gain[1])
        parts.append((m, O, l))
    M = np.max([m for m, _, _ in parts], axis=0)
    num = sum(np.exp2(m - M) * O for m, O, _ in parts)
    den = sum(np.exp2(m - M) * l for m, _, l in parts)
    return kr.bf16(num / den)


@pytest.mark.parametrize("sharp", [False, True])
def test_bf16_model_check_accepts_kernel_arithmetic_and_rejects_planted_bugs(sharp):
    q, K, V, scale = _inputs(sharp)
    sl2 = kr.scale_log2(scale, D)
    vis = np.ones((q.shape[0], K.shape[0]), dtype=bool)
    model, extra = kr.bf16_attention(q, K, V, vis, sl2)
    exact = oattn.softmax_attention(q, K, V, vis, sl2 / kr.LOG2E)
    ok = _f32_bf16_kernel(q, K, V, sl2, splits=3)
    rel_ok, _ = kr.assert_matches_model(ok, model, "float32 kernel arithmetic", extra)
    rel_exact = np.linalg.norm(ok - exact) / np.linalg.norm(exact)
    bugs = {"tile dropped": _f32_bf16_kernel(q, K, V, sl2, drop=(5 * T + 640, 5 * T + 704), splits=3),
            "split x1.05": _f32_bf16_kernel(q, K, V, sl2, splits=3, split_gain=(1, 1.05))}
    for name, got in bugs.items():
        rel, excess, _ = kr.model_mismatch(got, model, extra)
        assert rel > kr.MODEL_REL or excess > 0.0, f"{name} passes the model check (rel {rel:.2e})"
        # a bug is many times the correct arithmetic's distance from the model, while against the exact
        # oracle the correct arithmetic already sits at a good part of the bf16 tolerance
        assert rel > 10 * rel_ok, name
    assert rel_exact > 1.5e-3 if sharp else rel_exact > 5e-4


def _f32_e4m3_kernel(q_rot, K8, V8, qmul, v_scale, splits, drop=None, split_gain=None):
    """The e4m3 kernel's arithmetic in float32 (per-frame 64-key tiles, lazy integer max, splits)."""
    q8, e, _ = kr.q_e4m3(q_rot, qmul)
    sc = np.exp2(e.astype(np.float32))[:, None]
    s_all = ((q8.astype(np.float32) @ K8.astype(np.float32).T) * sc
             + _score_noise(q8, K8, seed=12) * sc)
    if drop is not None:
        s_all[:, drop[0]:drop[1]] = -np.inf
    ntf = (T + 63) // 64
    n_tiles = N_FR * ntf
    parts = []
    for sp in range(splits):
        lo, hi = n_tiles * sp // splits, n_tiles * (sp + 1) // splits
        m = np.full(q8.shape[0], -np.inf, dtype=np.float32)
        O = np.zeros((q8.shape[0], D), dtype=np.float32)
        l = np.zeros(q8.shape[0], dtype=np.float32)
        for kt in range(lo, hi):
            lf, j0 = kt // ntf, (kt % ntf) * 64
            keys = np.arange(lf * T + j0, lf * T + min(j0 + 64, T))
            st = s_all[:, keys]
            mx = st.max(axis=1)
            r = mx > m + 8
            mn = np.where(r, np.ceil(np.where(r, mx, 0)), m).astype(np.float32)
            a = np.where(r & np.isfinite(m), np.exp2(np.where(np.isfinite(m), m, 0) - mn), 1).astype(np.float32)
            O *= a[:, None]
            l *= a
            m = mn
            p = ofp8.round_e4m3(np.exp2(st - np.where(np.isfinite(m), m, 0)[:, None])).astype(np.float32)
            O += p @ V8[keys].astype(np.float32)
            l += p.sum(axis=1, dtype=np.float32)
        if split_gain is not None and sp == split_gain[0]:
            O *= np.float32(split_gain[1])
        parts.append((m, O * np.float32(v_scale), l))
    M = np.max([m for m, _, _ in parts], axis=0)
    num = sum(np.exp2(m - M)[:, None] * O for m, O, _ in parts)
    den = sum(np.exp2(m - M) * l for m, _, l in parts)
    return kr.bf16(num / den[:, None])


def test_e4m3_model_check_accepts_kernel_arithmetic_and_rejects_planted_bugs():
    q, K, V, _ = _inputs(False, seed=1)
    ks, vs = 1.0 / 64, 1.0 / 64
    K8 = ofp8.round_e4m3(K / ks)
    V8 = ofp8.round_e4m3(V / vs)
    qmul = float(np.float32(np.float32(kr.scale_log2(0.0, D)) * np.float32(ks)))
    fend = np.full(q.shape[0], N_FR)
    model, extra = kr.e4m3_attention(q, K8, V8, T, fend, fend, 3, qmul, vs)
    exact = oattn.softmax_attention(q, K, V, np.ones((q.shape[0], K.shape[0]), bool), 1.0 / np.sqrt(D))
    ok = _f32_e4m3_kernel(q, K8, V8, qmul, vs, 3)
    # the noisy scores do flip some e4m3 roundings: without the near-tie allowance the check would fail
    assert kr.model_mismatch(ok, model)[1] > 0.0
    kr.assert_matches_model(ok, model, "float32 e4m3 kernel arithmetic", extra)
    rel_ok_exact = np.linalg.norm(ok - exact) / np.linalg.norm(exact)
    for name, got in {"tile dropped": _f32_e4m3_kernel(q, K8, V8, qmul, vs, 3, drop=(7 * T + 64, 7 * T + 128)),
                      "split x1.05": _f32_e4m3_kernel(q, K8, V8, qmul, vs, 3, split_gain=(2, 1.05))}.items():
        rel, excess, _ = kr.model_mismatch(got, model, extra)
        assert rel > kr.MODEL_REL or excess > 0.0, f"{name} passes the model check (rel {rel:.2e})"
        rel_exact = np.linalg.norm(got - exact) / np.linalg.norm(exact)
        # against the exact oracle the bug hides inside the e4m3 rounding noise of a correct kernel
        assert rel_exact < 2.5 * rel_ok_exact, name
