"""GPU parity: sa_rope3d_apply, sa_cache_append (slot map, rotated K, V bits), sa_cache_read."""
import numpy as np
import pytest

import workloads as wl
from oracle import cache as ocache
from oracle import rope as orope
from swk_testutil import assert_close, log, to_dev, to_np, torch_dtype

pytestmark = pytest.mark.gpu


def _swk():
    import sink_window_kv_amd as swk
    return swk


def _rope_for(w, eps=None, jitter_axes=1):
    swk = _swk()
    return swk.Rope(w.n_heads, w.head_dim, w.dims, w.grid, w.theta0, w.sigma, eps, jitter_axes)


@pytest.mark.parametrize("cfg,t0,n_frames", [(1, 0, 3), (2, 5, 1), (3, 1198, 3), (3, 100000, 1)])
def test_rope3d_apply_matches_oracle(cfg, t0, n_frames):
    import torch
    swk = _swk()
    w = wl.WORKLOADS[cfg]
    log(f"rope3d cfg{cfg} t0={t0} n_frames={n_frames}")
    eps = wl.head_jitter(w) if w.sigma > 0 else None
    rope = _rope_for(w, eps)
    x = wl.chunk_qkv(w, 0, n_frames, tensor=wl.TENSOR_Q, scale=1.0)
    tx = to_dev(x, w.dtype)
    ty = torch.empty_like(tx)
    swk.sa_rope3d_apply(rope, tx, ty, w.batch, n_frames, t0)
    torch.cuda.synchronize()
    bases = orope.theta_hat(w.theta0, w.sigma, eps if eps is not None else np.zeros(w.n_heads))
    ref = orope.rope3d(x, t0, w.tokens_per_frame, bases, w.dims, w.grid[1])
    rel, mx = assert_close(to_np(ty), ref, w.dtype, f"rope cfg{cfg}")
    log(f"  rel_l2 {rel:.2e} max_abs {mx:.2e}")
    # in place (y aliases x) gives the same bits
    swk.sa_rope3d_apply(rope, tx, tx, w.batch, n_frames, t0)
    torch.cuda.synchronize()
    assert torch.equal(tx, ty)


@pytest.mark.parametrize("cfg,t0,t_scale", [(1, 5, 0.125), (3, 1198, 0.3), (3, 100000, 1.0 / 3.0)])
def test_rope3d_apply_position_interpolation(cfg, t0, t_scale):
    """Time positions t * t_scale (LoL review's PI baseline) against the oracle at fractional positions."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[cfg]
    eps = wl.head_jitter(w) if w.sigma > 0 else None
    rope = swk.Rope(w.n_heads, w.head_dim, w.dims, w.grid, w.theta0, w.sigma, eps, t_scale=t_scale)
    x = wl.chunk_qkv(w, 0, 2, tensor=wl.TENSOR_K, scale=1.0)
    tx = to_dev(x, w.dtype)
    ty = torch.empty_like(tx)
    swk.sa_rope3d_apply(rope, tx, ty, w.batch, 2, t0)
    torch.cuda.synchronize()
    bases = orope.theta_hat(w.theta0, w.sigma, eps if eps is not None else np.zeros(w.n_heads))
    ref = orope.rope3d(x, t0, w.tokens_per_frame, bases, w.dims, w.grid[1], t_scale=t_scale)
    rel, mx = assert_close(to_np(ty), ref, w.dtype, f"rope PI cfg{cfg}")
    log(f"  PI {t_scale:.3f} cfg{cfg} t0={t0}: rel_l2 {rel:.2e} max_abs {mx:.2e}")


def test_rope_theta_table_arbitrary_per_axis_bases():
    """theta_hat given as a per-head, per-axis table (LoL review, method steps (4)-(6)) with a different base
    on every axis of every head: the standalone rotation at large t, then a jittered Wan-1.3B stream (append
    rotates K with the table, the attention rotates q) on sampled rows, both against the oracle fed the same
    table."""
    import torch
    from test_gpu_attn import GpuStream, _check
    swk = _swk()
    w = wl.WORKLOADS[3]
    bases = np.random.default_rng(21).uniform(300.0, 30000.0, size=(w.n_heads, 3))
    rope = swk.Rope(w.n_heads, w.head_dim, w.dims, w.grid, theta=bases)
    x = wl.chunk_qkv(w, 3, 2, tensor=wl.TENSOR_Q, scale=1.0)
    tx = to_dev(x, "bf16")
    ty = torch.empty_like(tx)
    swk.sa_rope3d_apply(rope, tx, ty, 1, 2, 1199)
    torch.cuda.synchronize()
    rel, mx = assert_close(to_np(ty), orope.rope3d(x, 1199, w.tokens_per_frame, bases, w.dims, w.grid[1]),
                           "bf16", "rope theta table")
    log(f"  rope with a per-axis theta table: rel_l2 {rel:.2e} max_abs {mx:.2e}")
    gs = GpuStream(w, theta=bases)
    rows = np.arange(0, w.tokens_per_frame, 37)
    for f in range(13):
        q, k, v = (wl.frame_qkv(w, f, tensor=t, scale=None if t == wl.TENSOR_V else 1.0)
                   for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
        gs.append(k, v, 1, 50 * f)
        if f in (0, 12):
            o = gs.attend(q, 1, swk.SA_MASK_FRAME_CAUSAL)
            _check(gs, q, o, True, rows=rows, what=f"theta table frame {f} (t = {50 * f})")


def test_rope3d_apply_rejects_partial_overlap():
    """y must be x itself or disjoint from it: a shifted y is SA_ERR_RANGE, and nothing is written."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[1]
    rope = _rope_for(w)
    n = w.batch * w.tokens_per_frame * w.n_heads * w.head_dim
    buf = torch.zeros(2 * n, dtype=torch.float32, device="cuda")
    x = buf[:n]
    y = buf[w.head_dim:w.head_dim + n]       # starts inside x
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_rope3d_apply(rope, x, y, w.batch, 1, 3)
    assert e.value.status == swk.SA_ERR_RANGE
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(buf)) == 0


def test_rope_all_axes_jittered_and_host_tables():
    """Host tables equal the oracle's theta_hat/frequencies; all-axis jitter parity on device."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[3]
    eps = wl.head_jitter(w)
    th, fr = swk.sa_rope_tables(w.n_heads, w.head_dim, w.dims, w.grid, w.theta0, w.sigma, eps, 7)
    bases = orope.theta_hat(w.theta0, w.sigma, eps, jitter_axes=("t", "h", "w"))
    np.testing.assert_allclose(np.array(th), bases, rtol=1e-15)
    for h in range(w.n_heads):
        np.testing.assert_allclose(fr[h], orope.head_frequencies(bases[h], w.dims), rtol=1e-14)
    rope = _rope_for(w, eps, jitter_axes=7)
    x = wl.chunk_qkv(w, 7, 1, tensor=wl.TENSOR_K, scale=1.0)
    tx = to_dev(x, "bf16")
    ty = torch.empty_like(tx)
    swk.sa_rope3d_apply(rope, tx, ty, 1, 1, 777)
    torch.cuda.synchronize()
    ref = orope.rope3d(x, 777, w.tokens_per_frame, bases, w.dims, w.grid[1])
    assert_close(to_np(ty), ref, "bf16", "rope all-axes")


@pytest.mark.parametrize("cfg,chunk,frames", [(1, 1, 6), (2, 1, 14), (5, 3, 15), (2, 2, 8)])
def test_append_slots_k_v_match_oracle(cfg, chunk, frames):
    """Slot map exact vs the oracle model; V bit-exact; K within tolerance; fused == standalone RoPE bits."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[cfg]
    log(f"append cfg{cfg} chunk={chunk} frames={frames}")
    eps = wl.head_jitter(w) if w.sigma > 0 else None
    rope = _rope_for(w, eps)
    cache = swk.Cache(rope, w.batch, w.n_sink, w.n_local, torch_dtype(w.dtype))
    model = ocache.CacheModel(w.n_sink, w.n_local)
    bases = orope.theta_hat(w.theta0, w.sigma, eps if eps is not None else np.zeros(w.n_heads))
    kept = {}
    T = w.tokens_per_frame
    for f0 in range(0, frames, chunk):
        t0 = 10 + 2 * f0  # increasing, consecutive inside a chunk
        k = wl.chunk_qkv(w, f0, chunk, tensor=wl.TENSOR_K)
        v = wl.chunk_qkv(w, f0, chunk, tensor=wl.TENSOR_V)
        swk.sa_cache_append(cache, to_dev(k, w.dtype), to_dev(v, w.dtype), chunk, t0)
        model.append(chunk, t0)
        for i in range(chunk):
            kept[f0 + i] = (k[:, i * T:(i + 1) * T], v[:, i * T:(i + 1) * T], t0 + i)
        for f in list(kept):
            if f not in model.resident():
                del kept[f]
        slots = swk.sa_cache_slots(cache)
        ref_slots = model.slots()
        assert [(s.frame, s.t, s.segment, s.slot) for s in slots] == \
               [(e.frame, e.t, e.segment, e.slot) for e in ref_slots]
        assert swk.sa_cache_counts(cache) == (model.n_appended, len(ref_slots))
    torch.cuda.synchronize()
    dt = torch_dtype(w.dtype)
    for idx, e in enumerate(model.slots()):
        k, v, t = kept[e.frame]
        ko = torch.empty((w.batch, T, w.n_heads, w.head_dim), dtype=dt, device="cuda")
        vo = torch.empty_like(ko)
        swk.sa_cache_read(cache, idx, ko, vo)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(vo.cpu().float().numpy(), v)  # V bit-exact
        ref = orope.rope3d_frame(k, t, bases, w.dims, w.grid[1])
        assert_close(to_np(ko), ref, w.dtype, f"cached K frame {e.frame}")
        # fused RoPE in append == standalone RoPE, bit for bit
        ks = torch.empty_like(ko)
        swk.sa_rope3d_apply(rope, to_dev(k, w.dtype), ks, w.batch, 1, t)
        torch.cuda.synchronize()
        assert torch.equal(ks, ko), f"fused vs standalone RoPE differ at frame {e.frame}"


def test_append_errors_leave_state_unchanged():
    import torch
    swk = _swk()
    w = wl.WORKLOADS[1]
    rope = _rope_for(w)
    cache = swk.Cache(rope, 1, w.n_sink, w.n_local, torch.float32)
    T = w.tokens_per_frame
    k = torch.zeros((1, 4 * T, w.n_heads, w.head_dim), device="cuda")
    swk.sa_cache_append(cache, k[:, :T], k[:, :T], 1, 5)
    before = [(s.frame, s.t) for s in swk.sa_cache_slots(cache)]
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_append(cache, k, k, 4, 9)  # 3 non-sink frames > n_local = 2
    assert e.value.status == swk.SA_ERR_RANGE
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_append(cache, k[:, :T], k[:, :T], 1, 5)  # time does not increase
    assert e.value.status == swk.SA_ERR_RANGE
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_read(cache, 3, k[:, :T], None)
    assert e.value.status == swk.SA_ERR_RANGE
    assert [(s.frame, s.t) for s in swk.sa_cache_slots(cache)] == before
    swk.sa_cache_reset(cache)
    assert swk.sa_cache_slots(cache) == [] and swk.sa_cache_counts(cache) == (0, 0)
    swk.sa_cache_append(cache, k[:, :T], k[:, :T], 1, 0)  # time restarts after reset
    assert swk.sa_cache_counts(cache) == (1, 1)
