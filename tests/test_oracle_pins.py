"""Pins for the fp64 oracle: closed forms, invariants, library routines, brute force.

Each test names the fact it pins and the passage that fixes it.  A
plausible slip in the oracle (dropped scale, wrong rotation sign, wrong
frequency index, swapped axis, wrong eviction) fails at least one test.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import brute, cache as ocache, diagnostics as odiag, fp8 as ofp8, project as oproject, quant as oquant, recache as orecache, rope as orope, stream as ostream

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _tiny_setup(sigma=0.8, H=2, dims=(4, 2, 2), grid=(2, 2)):
    eps = RNG.uniform(-1, 1, size=H)
    bases = orope.theta_hat(10000.0, sigma, eps)
    return bases, dims, grid


# ---------------------------------------------------------------- P1 brute force
@pytest.mark.parametrize("chunks", [[1, 1, 1, 1, 1], [2, 2, 1], [1, 2, 2]])
def test_p1_brute_force_stream_matches_numpy(chunks):
    """Pure-Python loops vs the numpy oracle, whole stream, 1e-12 (brute force on tiny inputs)."""
    bases, dims, grid = _tiny_setup()
    T = grid[0] * grid[1]
    H, D = 2, sum(dims)
    n = sum(chunks)
    q = RNG.standard_normal((n, 1, T, H, D))
    k = RNG.standard_normal((n, 1, T, H, D))
    v = RNG.standard_normal((n, 1, T, H, D))
    times = [f + 5 for f in range(n)]   # consecutive: append gives frame i of a chunk t0 + i
    ref = brute.stream_attention([q[f, 0].tolist() for f in range(n)],
                                 [k[f, 0].tolist() for f in range(n)],
                                 [v[f, 0].tolist() for f in range(n)],
                                 times, 1, 2, bases.tolist(), dims, grid[1], causal_chunks=chunks)
    so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases)
    f0 = 0
    for c in chunks:
        kk = np.concatenate([k[f] for f in range(f0, f0 + c)], axis=1)
        vv = np.concatenate([v[f] for f in range(f0, f0 + c)], axis=1)
        qq = np.concatenate([q[f] for f in range(f0, f0 + c)], axis=1)
        so.append(kk, vv, times[f0])
        o = so.attend(qq, causal=True)
        for i in range(c):
            np.testing.assert_allclose(o[0, i * T:(i + 1) * T], np.array(ref[f0 + i]), rtol=0, atol=1e-12)
        f0 += c


def test_p1_brute_force_rope_and_projection():
    bases, dims, grid = _tiny_setup(H=3)
    T = grid[0] * grid[1]
    x = RNG.standard_normal((1, T, 3, sum(dims)))
    out = orope.rope3d_frame(x, 17, bases, dims, grid[1])
    for tok in range(T):
        for h in range(3):
            ref = brute.rope_vector(x[0, tok, h].tolist(), brute.positions(17, tok, grid[1], dims),
                                    brute.frequencies(bases[h], dims))
            np.testing.assert_allclose(out[0, tok, h], ref, rtol=0, atol=1e-13)
    xs = RNG.standard_normal((1, 5, 6))
    w = RNG.standard_normal((6, 4))
    np.testing.assert_allclose(orecache.project(xs, w, 2).reshape(5, 4),
                               brute.matvec_rows(xs[0].tolist(), w.tolist()), rtol=0, atol=1e-12)


# ------------------------------------------- P2 window covering everything = full attention
@pytest.mark.parametrize("chunk", [1, 2])
def test_p2_window_covering_all_frames_is_full_causal_attention(chunk):
    """n_sink + n_local >= frames streamed => exactly block-causal full attention (torch SDPA, fp64)."""
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 3))
    T, H, D = grid[0] * grid[1], 2, 8
    n = 6
    q = RNG.standard_normal((1, n * T, H, D))
    k = RNG.standard_normal((1, n * T, H, D))
    v = RNG.standard_normal((1, n * T, H, D))
    so = ostream.StreamOracle(2, 4, T, grid[1], dims, bases)
    outs = []
    for f0 in range(0, n, chunk):
        sl = slice(f0 * T, (f0 + chunk) * T)
        so.append(k[:, sl], v[:, sl], f0)
        outs.append(so.attend(q[:, sl], causal=True))
    got = np.concatenate(outs, axis=1)
    # library routine on the whole sequence
    qr = orope.rope3d(q, 0, T, bases, dims, grid[1])
    kr = orope.rope3d(k, 0, T, bases, dims, grid[1])
    fr = np.repeat(np.arange(n), T)
    # a query of frame f sees frames <= f (frame-causal) -- inside a chunk and across chunks
    mask = torch.from_numpy(fr[None, :] <= fr[:, None])
    tq = torch.from_numpy(qr).permute(0, 2, 1, 3)
    tk = torch.from_numpy(kr).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_p2_non_causal_mode_sees_whole_window():
    bases, dims, grid = _tiny_setup(H=1, dims=(4, 2, 2), grid=(1, 2))
    T, D = 2, 8
    so = ostream.StreamOracle(1, 3, T, grid[1], dims, bases)
    k = RNG.standard_normal((1, 3 * T, 1, D))
    v = RNG.standard_normal((1, 3 * T, 1, D))
    q = RNG.standard_normal((1, 3 * T, 1, D))
    so.append(k, v, 0)
    got = so.attend(q, causal=False)
    qr = orope.rope3d(q, 0, T, bases, dims, grid[1])
    kr = orope.rope3d(k, 0, T, bases, dims, grid[1])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr).permute(0, 2, 1, 3), torch.from_numpy(kr).permute(0, 2, 1, 3),
        torch.from_numpy(v).permute(0, 2, 1, 3))
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ P3 relative position
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_p3_scores_depend_only_on_offset(axis):
    """<R(m)q, R(n)k> = <q, R(n-m)k> on each axis and for each jittered head (LoL review, RoPE)."""
    bases, dims, _ = _tiny_setup(H=3, dims=(6, 4, 4))
    D = sum(dims)
    q = RNG.standard_normal(D)
    k = RNG.standard_normal(D)
    for h in range(3):
        w = orope.head_frequencies(bases[h], dims)
        seg = np.zeros(D // 2)
        start = sum(dims[:axis]) // 2
        seg[start:start + dims[axis] // 2] = 1.0
        for m, n in [(0, 5), (7, 12), (300, 305), (1200, 1205)]:
            qm = orope.rotate_pairs(q, m * seg * w)
            kn = orope.rotate_pairs(k, n * seg * w)
            rel = orope.rotate_pairs(k, (n - m) * seg * w)
            assert abs(qm @ kn - q @ rel) < 1e-9
        # same offset, different absolute positions -> same score
        s1 = orope.rotate_pairs(q, 3 * seg * w) @ orope.rotate_pairs(k, 10 * seg * w)
        s2 = orope.rotate_pairs(q, 903 * seg * w) @ orope.rotate_pairs(k, 910 * seg * w)
        assert abs(s1 - s2) < 1e-9


def test_p3_time_shift_leaves_stream_output_unchanged():
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 2))
    T, D = 4, 8
    q = RNG.standard_normal((1, 4 * T, 2, D))
    k = RNG.standard_normal((1, 4 * T, 2, D))
    v = RNG.standard_normal((1, 4 * T, 2, D))
    outs = []
    for shift in (0, 1000):
        so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases)
        o = None
        for f in range(4):
            sl = slice(f * T, (f + 1) * T)
            so.append(k[:, sl], v[:, sl], f + shift)
            o = so.attend(q[:, sl], causal=True)
        outs.append(o)
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-10)


# ------------------------------------------------------------ P4 sigma = 0 is textbook RoPE
def test_p4_sigma_zero_is_textbook_rope_complex_form():
    """sigma = 0 (or eps = 0) reduces to standard RoPE: (x0 + i x1) * exp(i pos theta^(-2j/d))."""
    dims, grid_w = (44, 42, 42), 52
    H, D = 3, 128
    b0 = orope.theta_hat(10000.0, 0.0, RNG.uniform(-1, 1, H))
    b1 = orope.theta_hat(10000.0, 0.8, np.zeros(H))
    np.testing.assert_array_equal(b0, b1)
    x = RNG.standard_normal((1, 1560, H, D))
    got = orope.rope3d_frame(x, 37, b0, dims, grid_w)
    tok = np.arange(1560)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    ang = []
    for a, pos in enumerate([np.full(1560, 37.0), tok // grid_w, tok % grid_w]):
        inv = 1.0 / (10000.0 ** (np.arange(0, dims[a], 2) / dims[a]))
        ang.append(np.outer(pos, inv))
    ang = np.concatenate(ang, axis=1)
    zr = z * np.exp(1j * ang)[None, :, None, :]
    ref = np.empty_like(x)
    ref[..., 0::2] = zr.real
    ref[..., 1::2] = zr.imag
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_p4_rotation_direction_and_frequency_index():
    """Pair 0 turns by exactly pos radians (exponent 0); (1,0) at pi/2 goes to (0,1) (counter-clockwise)."""
    w = orope.axis_frequencies(12345.0, 8)
    assert w[0] == 1.0
    np.testing.assert_allclose(w[1:], [12345.0 ** (-0.25), 12345.0 ** (-0.5), 12345.0 ** (-0.75)], rtol=1e-15)
    out = orope.rotate_pairs(np.array([1.0, 0.0]), np.array([np.pi / 2]))
    np.testing.assert_allclose(out, [0.0, 1.0], atol=1e-16)
    # 3D: token 0 at t = 0 is the identity; frequencies of the h/w segments restart at 1
    x = RNG.standard_normal((1, 1, 1, 8))
    b = orope.theta_hat(10000.0, 0.0, [0.0])
    np.testing.assert_array_equal(orope.rope3d_frame(x, 0, b, (4, 2, 2), 3), x)
    f = orope.head_frequencies(b[0], (4, 2, 2))
    np.testing.assert_allclose(f, [1.0, 0.01, 1.0, 1.0])


def test_p4_lol_bases_match_page_parameters():
    """theta0 = 10000, sigma = 0.8, eps in U[-1,1]: eps=-1,0,1 give 2000, 10000, 18000 (golden)."""
    vals = {}
    for line in open(os.path.join(GOLDEN, "lol_setup.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, val = line.split()
        vals[key] = float(val)
    b = orope.theta_hat(vals["theta0"], vals["sigma"], [-1.0, 0.0, 1.0])
    np.testing.assert_allclose(b[:, 0], [vals["theta_hat_at_eps_minus1"], vals["theta_hat_at_eps_0"],
                                         vals["theta_hat_at_eps_plus1"]], rtol=1e-15)
    np.testing.assert_array_equal(b[:, 1:], vals["theta0"])  # spatial axes are not jittered
    ball = orope.theta_hat(10000.0, 0.8, [1.0], jitter_axes=("t", "h", "w"))
    np.testing.assert_allclose(ball, [[18000.0] * 3])


# ------------------------------------------------------------ P5 softmax normalisation
def test_p5_probabilities_are_normalised():
    q = RNG.standard_normal((7, 16)) * 3
    k = RNG.standard_normal((40, 16)) * 3
    v = RNG.standard_normal((40, 16))
    vis = RNG.random((7, 40)) < 0.5
    vis[:, 0] = True
    o, p = oattn.softmax_attention(q, k, v, vis, 0.25, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert (p >= 0).all() and (p[~vis] == 0).all()
    np.testing.assert_allclose(o, p @ v, atol=1e-12)
    # the scale enters: doubling it equals doubling q
    o2 = oattn.softmax_attention(2 * q, k, v, vis, 0.25)
    o3 = oattn.softmax_attention(q, k, v, vis, 0.5)
    np.testing.assert_allclose(o2, o3, atol=1e-12)
    # library routine: torch softmax in fp64
    s = torch.from_numpy((q @ k.T) * 0.25).masked_fill(torch.from_numpy(~vis), float("-inf"))
    np.testing.assert_allclose(p, torch.softmax(s, dim=1).numpy(), atol=1e-14)


# ------------------------------------------------------------ P6 recache idempotence
def test_p6_recache_with_unchanged_weights_reproduces_cache():
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 2))
    T, H, D, C = 4, 2, 8, 12
    w_k = RNG.standard_normal((C, H * D)) / math.sqrt(C)
    w_v = RNG.standard_normal((C, H * D)) / math.sqrt(C)
    so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases)
    xs = {}
    for f in range(5):
        x = RNG.standard_normal((1, T, C))
        xs[f] = x
        k = orecache.project(x, w_k, H)
        v = orecache.project(x, w_v, H)
        so.append(k, v, 10 + f)
    res = so.resident()
    before = {f: so.frame_kv(f) for f in res}
    x_all = np.concatenate([xs[f] for f in res], axis=1)
    so.recache(x_all, w_k, w_v)
    for f in res:
        np.testing.assert_allclose(so.frame_kv(f)[0], before[f][0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(so.frame_kv(f)[1], before[f][1], rtol=0, atol=1e-13)
    assert so.resident() == res
    # with new weights the values are exactly x . W_new (library matmul)
    w_new = RNG.standard_normal((C, H * D))
    so.recache(x_all, w_k, w_new)
    for j, f in enumerate(res):
        np.testing.assert_allclose(so.frame_kv(f)[1][0].reshape(T, H * D),
                                   torch.from_numpy(x_all[0, j * T:(j + 1) * T]) .matmul(torch.from_numpy(w_new)).numpy(),
                                   atol=1e-12)


# ------------------------------------------------------------ P9 projections
def _perm_matrix(perm):
    """Column-selection matrix: (x . P)[..., j] = x[..., perm[j]]."""
    n = len(perm)
    p = np.zeros((n, n))
    for j, i in enumerate(perm):
        p[i, j] = 1.0
    return p


def test_p9_linear_matches_brute_force_and_selection():
    """x . W (LoL paper review, background "multi-head attention" projections): brute-force loops on a
    non-square W, and a selection matrix picks columns (a transposed W would pick the inverse permutation)."""
    x = RNG.standard_normal((2, 5, 6))
    w = RNG.standard_normal((6, 4))
    y = oproject.linear(x, w)
    assert y.shape == (2, 5, 4)
    for b in range(2):
        np.testing.assert_allclose(y[b], brute.matvec_rows(x[b].tolist(), w.tolist()), rtol=0, atol=1e-12)
    perm = [2, 0, 5, 1, 3, 4]     # not its own inverse
    np.testing.assert_array_equal(oproject.linear(x, _perm_matrix(perm)), x[..., perm])
    np.testing.assert_array_equal(oproject.linear(x, np.eye(6)), x)


def test_p9_project_append_with_selection_weights_is_plain_append():
    """With permutation weights the projections reduce to appending the permuted inputs: same cache,
    same slots, same evictions, q = the permuted x (the append path is pinned by P3, P4 and P8)."""
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 2))
    T, H, D = 4, 2, 8
    C = H * D
    pq, pk, pv = (list(RNG.permutation(C)) for _ in range(3))
    a = ostream.StreamOracle(1, 3, T, grid[1], dims, bases)
    b = ostream.StreamOracle(1, 3, T, grid[1], dims, bases)
    t0 = 3
    for c in (1, 2, 1, 3, 2):
        x = RNG.standard_normal((2, c * T, C))
        q, ev_a = oproject.project_append(a, x, _perm_matrix(pq), _perm_matrix(pk), _perm_matrix(pv), H, t0)
        ev_b = b.append(x[..., pk].reshape(2, c * T, H, D), x[..., pv].reshape(2, c * T, H, D), t0)
        assert ev_a == ev_b
        np.testing.assert_array_equal(q, x[..., pq].reshape(2, c * T, H, D))
        assert a.resident() == b.resident()
        for f in a.resident():
            np.testing.assert_array_equal(a.frame_kv(f)[0], b.frame_kv(f)[0])
            np.testing.assert_array_equal(a.frame_kv(f)[1], b.frame_kv(f)[1])
        t0 += c + 2
    q, _ = oproject.project_append(a, RNG.standard_normal((2, T, C)), None, np.eye(C), np.eye(C), H, t0)
    assert q is None


def test_p9_project_append_brute_force():
    """Brute-force loops: q = x W_q, K = RoPE(x W_k, t_f) per head and token, V = x W_v."""
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 2))
    T, H, D, C = 4, 2, 8, 5
    w_q, w_k, w_v = (RNG.standard_normal((C, H * D)) for _ in range(3))
    so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases)
    x = RNG.standard_normal((1, 2 * T, C))
    t0 = 7
    q, _ = oproject.project_append(so, x, w_q, w_k, w_v, H, t0)
    qb = brute.matvec_rows(x[0].tolist(), w_q.tolist())
    kb = brute.matvec_rows(x[0].tolist(), w_k.tolist())
    vb = brute.matvec_rows(x[0].tolist(), w_v.tolist())
    np.testing.assert_allclose(q[0].reshape(2 * T, H * D), qb, rtol=0, atol=1e-12)
    for j, f in enumerate(so.resident()):
        kf, vf = so.frame_kv(f)
        for tok in range(T):
            row = j * T + tok
            np.testing.assert_allclose(vf[0, tok].reshape(H * D), vb[row], rtol=0, atol=1e-12)
            for h in range(H):
                ref = brute.rope_vector(kb[row][h * D:(h + 1) * D], brute.positions(t0 + j, tok, grid[1], dims),
                                        brute.frequencies(bases[h], dims))
                np.testing.assert_allclose(kf[0, tok, h], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------ P10 LoL diagnostics
@pytest.mark.parametrize("causal", [True, False])
def test_p10_sink_mass_brute_force(causal):
    """Sink mass = the brute-force attention row of 0/1 values marking the sink keys (pure-Python loops)."""
    bases, dims, grid = _tiny_setup()
    T, H, D = 4, 2, 8
    so = ostream.StreamOracle(2, 2, T, grid[1], dims, bases)
    for f in range(6):
        so.append(RNG.standard_normal((1, T, H, D)), RNG.standard_normal((1, T, H, D)), 3 + f)
    q = RNG.standard_normal((1, 2 * T, H, D)) * 2.0
    mass = odiag.sink_mass(so, q, causal)
    res = so.resident()
    qframes = res[-2:]
    for i, fq in enumerate(qframes):
        for tok in range(T):
            for h in range(H):
                qv = brute.rope_vector(q[0, i * T + tok, h].tolist(),
                                       brute.positions(so.model.t[fq], tok, grid[1], dims),
                                       brute.frequencies(bases[h], dims))
                keys, marks = [], []
                for fk in res:
                    if causal and fk > fq:
                        continue
                    for kt in range(T):
                        keys.append(so.frame_kv(fk)[0][0, kt, h].tolist())
                        marks.append([1.0 if fk < 2 else 0.0])
                ref = brute.attention_row(qv, keys, marks, 1.0 / math.sqrt(D))[0]
                assert abs(mass[0, i * T + tok, h] - ref) <= 1e-12


def test_p10_sink_mass_closed_forms():
    """No sinks -> 0; a query frame that is itself a sink sees only sinks -> 1; q = 0 -> the share of
    visible sink keys."""
    bases, dims, grid = _tiny_setup()
    T, H, D = 4, 2, 8
    none = ostream.StreamOracle(0, 3, T, grid[1], dims, bases)
    both = ostream.StreamOracle(2, 3, T, grid[1], dims, bases)
    for f in range(5):
        k, v = RNG.standard_normal((1, T, H, D)), RNG.standard_normal((1, T, H, D))
        none.append(k, v, f)
        both.append(k, v, f)
        q = RNG.standard_normal((1, T, H, D))
        assert np.all(odiag.sink_mass(none, q, True) == 0.0)
        m = odiag.sink_mass(both, q, True)
        if f < 2:
            np.testing.assert_allclose(m, 1.0, rtol=0, atol=1e-15)
        visible = len(both.resident())
        np.testing.assert_allclose(odiag.sink_mass(both, np.zeros_like(q), True), min(f + 1, 2) / visible,
                                   rtol=0, atol=1e-15)


def test_p10_phase_coherence():
    """C(0) = 1; |C| <= 1; sigma = 0 -> every head equal; d_t = 2 -> C = exp(j Delta) (w_0 = 1);
    brute-force cos/sin loops over the time frequencies."""
    deltas = [0, 1, 3, 132, 201, 1200]
    eps = RNG.uniform(-1, 1, size=4)
    bases = orope.theta_hat(10000.0, 0.8, eps)
    dims = (44, 42, 42)
    c = odiag.phase_coherence(bases, dims, deltas)
    np.testing.assert_allclose(c[:, 0], 1.0, atol=1e-15)
    assert np.all(np.abs(c) <= 1.0 + 1e-12)
    assert np.abs(c[0] - c[1]).max() > 1e-3          # jitter separates the heads
    flat = odiag.phase_coherence(orope.theta_hat(10000.0, 0.0, eps), dims, deltas)
    np.testing.assert_allclose(flat, np.broadcast_to(flat[0], flat.shape), rtol=0, atol=0)
    one = odiag.phase_coherence(bases, (2, 4, 2), deltas)
    np.testing.assert_allclose(one, np.exp(1j * np.array(deltas, dtype=float))[None, :].repeat(4, 0), atol=1e-12)
    for h in range(4):
        w = brute.frequencies(bases[h], dims)[:dims[0] // 2]
        for n, dl in enumerate(deltas):
            re = sum(math.cos(x * dl) for x in w) / len(w)
            im = sum(math.sin(x * dl) for x in w) / len(w)
            assert abs(c[h, n].real - re) <= 1e-12 and abs(c[h, n].imag - im) <= 1e-12


# ------------------------------------------------------------ P11 e4m3 rounding
def test_p11_e4m3_codes_round_trip_and_known_values():
    """Every finite code decodes (from the bit fields) to a value that rounds to itself; the decoded
    values are strictly increasing from 0x00 to 0x7e; values fixed by the format definition."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = ofp8.decode(codes)
    np.testing.assert_array_equal(ofp8.round_e4m3(vals), vals)
    pos = ofp8.decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert ofp8.decode(0x38) == 1.0 and ofp8.decode(0x7E) == 448.0 and ofp8.decode(0x01) == 2.0 ** -9
    assert ofp8.decode(0x08) == 2.0 ** -6 and ofp8.decode(0x07) == 7 * 2.0 ** -9 and ofp8.decode(0xC0) == -2.0
    assert np.isnan(ofp8.decode(0x7F))


def test_p11_e4m3_ties_to_even_and_clamp():
    """Midpoints between neighbouring codes go to the code with an even mantissa; off-midpoint values go
    to the nearer code; magnitudes beyond 448 clamp to 448."""
    pos = ofp8.decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    got = ofp8.round_e4m3(mids)
    even = np.where(np.arange(0x7E) % 2 == 0, pos[:-1], pos[1:])   # code parity = mantissa parity
    np.testing.assert_array_equal(got, even)
    np.testing.assert_array_equal(ofp8.round_e4m3(-mids), -even)
    np.testing.assert_array_equal(ofp8.round_e4m3(mids - 1e-12 * pos[1:]), pos[:-1])
    np.testing.assert_array_equal(ofp8.round_e4m3(mids + 1e-12 * pos[1:]), pos[1:])
    np.testing.assert_array_equal(ofp8.round_e4m3([449.0, 1e9, -500.0]), [448.0, 448.0, -448.0])
    np.testing.assert_allclose(ofp8.quantize([3.0, 1000.0], 2.0), [3.0, 896.0])


# ------------------------------------------------------------ P12 position interpolation
def test_p12_pi_time_position_is_textbook_rope_at_fractional_position():
    """t_scale s: the time pairs turn by (s t) theta^(-2j/d_t), the grid pairs as without PI
    (textbook complex form at a fractional position; LoL review, PI baseline)."""
    dims, grid_w = (44, 42, 42), 52
    H, D, t, sc = 2, 128, 37, 0.3
    b = orope.theta_hat(10000.0, 0.0, np.zeros(H))
    x = RNG.standard_normal((1, 1560, H, D))
    got = orope.rope3d_frame(x, t, b, dims, grid_w, t_scale=sc)
    tok = np.arange(1560)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    ang = []
    for a, pos in enumerate([np.full(1560, t * sc), tok // grid_w, tok % grid_w]):
        inv = 1.0 / (10000.0 ** (np.arange(0, dims[a], 2) / dims[a]))
        ang.append(np.outer(pos, inv))
    zr = z * np.exp(1j * np.concatenate(ang, axis=1))[None, :, None, :]
    ref = np.empty_like(x)
    ref[..., 0::2] = zr.real
    ref[..., 1::2] = zr.imag
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(orope.rope3d_frame(x, t, b, dims, grid_w, t_scale=1.0),
                                  orope.rope3d_frame(x, t, b, dims, grid_w))


def test_p12_pi_compression_equals_stream_at_compressed_times():
    """A stream with t_scale 1/4 fed frames at t = 4f (appends, attention and a recache) gives the
    outputs of an uncompressed stream fed the same frames at t = f."""
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 2))
    T, D, C = 4, 8, 6
    q, k, v = (RNG.standard_normal((1, 6 * T, 2, D)) for _ in range(3))
    x = RNG.standard_normal((1, 3 * T, C))
    wk, wv = RNG.standard_normal((C, 2 * D)), RNG.standard_normal((C, 2 * D))
    outs = []
    for step, sc in ((1, 1.0), (4, 0.25)):
        so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases, t_scale=sc)
        o = []
        for f in range(6):
            sl = slice(f * T, (f + 1) * T)
            so.append(k[:, sl], v[:, sl], step * f)
            if f == 3:
                so.recache(x, wk, wv)
            o.append(so.attend(q[:, sl], causal=True))
        outs.append(np.concatenate(o, axis=1))
    np.testing.assert_allclose(outs[1], outs[0], rtol=0, atol=1e-12)
    # and it differs from the same t = 4f stream without PI
    so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases)
    for f in range(2):
        so.append(k[:, f * T:(f + 1) * T], v[:, f * T:(f + 1) * T], 4 * f)
    assert np.abs(so.attend(q[:, T:2 * T], causal=True) - outs[0][:, T:2 * T]).max() > 1e-3


def test_p12_pi_phase_coherence_scales_the_offset():
    """C(Delta) under t_scale s is C(s Delta) without it; d_t = 2 gives exp(j s Delta)."""
    eps = RNG.uniform(-1, 1, size=3)
    bases = orope.theta_hat(10000.0, 0.8, eps)
    deltas = np.array([0.0, 2.0, 10.0, 264.0, 402.0])
    np.testing.assert_allclose(odiag.phase_coherence(bases, (44, 42, 42), deltas, t_scale=0.5),
                               odiag.phase_coherence(bases, (44, 42, 42), deltas / 2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(odiag.phase_coherence(bases, (2, 4, 2), deltas, t_scale=0.125),
                               np.exp(1j * 0.125 * deltas)[None, :].repeat(3, 0), atol=1e-13)


# ------------------------------------------------------------ P13 8-bit projections
def test_p13_int8_rows_closed_forms():
    """Row max 127 gives scale 1 and codes = x rounded half to even; max 2 gives inv 63.5 (1 -> 63.5 -> 64);
    a zero row gives scale 0 and codes 0; the largest magnitude maps to +-127 exactly."""
    x = np.array([[127.0, 2.5, -3.5, 0.5, -127.0, 1.49], [2.0, 1.0, -0.5, 0.0, -2.0, 0.25], [0.0] * 6])
    c, sc = oquant.quantize_rows(x, "int8")
    assert c.dtype == np.int8 and sc.dtype == np.float32
    np.testing.assert_array_equal(c[0], [127, 2, -4, 0, -127, 1])
    np.testing.assert_array_equal(c[1], [127, 64, -32, 0, -127, 16])
    np.testing.assert_array_equal(c[2], 0)
    np.testing.assert_array_equal(sc, np.float32([1.0, 2.0 / 127.0, 0.0]))
    xr = RNG.standard_normal((40, 96)).astype(np.float32) * np.float32(3.0)
    c, sc = oquant.quantize_rows(xr, "int8")
    np.testing.assert_array_equal(np.abs(c).max(axis=1), 127)
    err = np.abs(xr - oquant.dequantize(c, sc, "int8"))
    assert np.all(err <= sc[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_p13_e4m3_rows_and_codes():
    """Every finite e4m3 code encodes back to itself (zeros keep their sign); a row with max 448 keeps its
    values rounded to e4m3 (448 -> 0x7e, 1 -> 0x38, -3 -> 0xc4); scaled rows put their max at 448 and
    stay within half an e4m3 step."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(oquant.e4m3_encode(ofp8.decode(codes)), codes)
    c, sc = oquant.quantize_rows(np.array([[448.0, 1.0, -3.0, 0.1, -1e-6]]), "e4m3")
    np.testing.assert_array_equal(c[0], [0x7E, 0x38, 0xC4, oquant.e4m3_encode(ofp8.round_e4m3(0.1)), 0x80])
    assert sc[0] == 1.0
    xr = RNG.standard_normal((30, 64)).astype(np.float32)
    c, sc = oquant.quantize_rows(xr, "e4m3")
    np.testing.assert_array_equal(np.abs(ofp8.decode(c)).max(axis=1), 448.0)
    y = xr.astype(np.float64) / sc[:, None]
    err = np.abs(y - ofp8.decode(c))
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-5))


@pytest.mark.parametrize("qtype", ["int8", "e4m3"])
def test_p13_linear_q8_brute_force(qtype):
    """The W8A8 product equals brute-force loops over the codes (x rows times weight rows, scales per
    x row and per weight row); for int8 the fp32 recipe is within 3 fp32 roundings of the exact value."""
    n, C, F = 5, 12, 7
    cx, sx = oquant.quantize_rows(RNG.standard_normal((n, C)), qtype)
    cw, sw = oquant.quantize_rows(RNG.standard_normal((F, C)) * 0.1, qtype)
    got = oquant.linear_q8(cx, sx, cw, sw, qtype)
    vx, vw = oquant.decode(cx, qtype), oquant.decode(cw, qtype)
    for i in range(n):
        for f in range(F):
            acc = 0.0
            for c in range(C):
                acc += float(vx[i, c]) * float(vw[f, c])
            ref = acc * float(sx[i]) * float(sw[f])
            assert abs(float(got[i, f]) - ref) <= 4 * 2.0 ** -24 * abs(ref) + 1e-30, (i, f)
    if qtype == "int8":
        assert got.dtype == np.float32
        acc = sum(int(cx[1, c]) * int(cw[2, c]) for c in range(C))
        assert got[1, 2] == (np.float32(acc) * sx[1]) * sw[2]


# ------------------------------------------------------------ P7 closed forms
def test_p7_single_visible_key_returns_its_value():
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(1, 1))
    so = ostream.StreamOracle(1, 2, 1, 1, dims, bases)
    k = RNG.standard_normal((1, 1, 2, 8))
    v = RNG.standard_normal((1, 1, 2, 8))
    q = RNG.standard_normal((1, 1, 2, 8)) * 10
    so.append(k, v, 0)
    np.testing.assert_allclose(so.attend(q, causal=True), v, atol=1e-14)


def test_p7_zero_query_averages_visible_values():
    bases, dims, grid = _tiny_setup(H=2, dims=(4, 2, 2), grid=(2, 2))
    T = 4
    so = ostream.StreamOracle(1, 2, T, grid[1], dims, bases)
    vs = []
    for f in range(5):
        k = RNG.standard_normal((1, T, 2, 8))
        v = RNG.standard_normal((1, T, 2, 8))
        vs.append(v)
        so.append(k, v, f)
    o = so.attend(np.zeros((1, T, 2, 8)), causal=True)
    mean = np.concatenate([vs[f] for f in so.resident()], axis=1).mean(axis=1)
    np.testing.assert_allclose(o, np.broadcast_to(mean[:, None], o.shape), atol=1e-14)


def test_p7_rotation_preserves_pair_norms_and_composes():
    x = RNG.standard_normal(16)
    a = RNG.standard_normal(8)
    b = RNG.standard_normal(8)
    y = orope.rotate_pairs(x, a)
    np.testing.assert_allclose(y[0::2] ** 2 + y[1::2] ** 2, x[0::2] ** 2 + x[1::2] ** 2, rtol=1e-13)
    np.testing.assert_allclose(orope.rotate_pairs(orope.rotate_pairs(x, a), b),
                               orope.rotate_pairs(x, a + b), atol=1e-13)


def test_p7_frame_order_does_not_matter_without_mask():
    """Ring order is irrelevant to the unmasked result: permuting the key frames leaves O unchanged."""
    T, H, D = 3, 2, 8
    q = RNG.standard_normal((1, T, H, D))
    ks = [RNG.standard_normal((1, T, H, D)) for _ in range(4)]
    vs = [RNG.standard_normal((1, T, H, D)) for _ in range(4)]
    o1 = oattn.window_attention(q, ks, vs, [0, 1, 2, 3], [3], T, causal=False)
    perm = [2, 0, 3, 1]
    o2 = oattn.window_attention(q, [ks[i] for i in perm], [vs[i] for i in perm], perm, [3], T, causal=False)
    np.testing.assert_allclose(o1, o2, atol=1e-14)


# ------------------------------------------------------------ P8 cache indexing
def _read_golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        f, res, ev, seg = [c.strip() for c in line.split("|")]
        rows.append((int(f), [int(x) for x in res.split()], [] if ev == "-" else [int(x) for x in ev.split()], seg))
    return rows


@pytest.mark.parametrize("name,n_sink,n_local,frames", [("cache_sink1_local2.txt", 1, 2, 6),
                                                         ("cache_sink3_local9.txt", 3, 9, 40)])
def test_p8_cache_matches_hand_derived_golden(name, n_sink, n_local, frames):
    golden = {r[0]: r for r in _read_golden(name)}
    m = ocache.CacheModel(n_sink, n_local)
    for f in range(frames):
        ev = m.append(1, f)
        if f in golden:
            _, res, gev, seg = golden[f]
            assert m.resident() == res
            assert ev == gev
            s, slot = ocache.slot_of(f, n_sink, n_local)
            assert seg == ("sink" if s == 0 else "ring") + ":" + str(slot)


@pytest.mark.parametrize("n_sink,n_local,chunk", [(1, 2, 1), (3, 9, 1), (3, 9, 3), (0, 4, 2), (2, 3, 3)])
def test_p8_cache_matches_deque_model(n_sink, n_local, chunk):
    """Independent model: a list of sinks plus collections.deque(maxlen=n_local)."""
    from collections import deque
    sinks, ring = [], deque(maxlen=n_local)
    m = ocache.CacheModel(n_sink, n_local)
    slots_ring = {}
    for f0 in range(0, 30, chunk):
        m.append(chunk, f0)
        for f in range(f0, f0 + chunk):
            if len(sinks) < n_sink:
                sinks.append(f)
            else:
                ring.append(f)
                slots_ring[f] = (len(slots_ring)) % n_local
        assert m.resident() == sinks + list(ring)
        for e in m.slots():
            if e.segment == 1:
                assert e.slot == slots_ring[e.frame]
            else:
                assert e.slot == e.frame


def test_p8_errors():
    m = ocache.CacheModel(3, 9)
    m.append(3, 0)
    with pytest.raises(ValueError):
        m.append(10, 3)       # chunk larger than the ring
    with pytest.raises(ValueError):
        m.append(1, 2)        # time does not increase
    m.reset()
    assert m.resident() == [] and m.n_appended == 0
