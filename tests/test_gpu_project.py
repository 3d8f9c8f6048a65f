"""GPU parity: sa_cache_project_append (per-frame Q/K/V projections + append) and sa_linear vs the fp64 oracle."""
import numpy as np
import pytest

import workloads as wl
from oracle import project as oproject
from swk_testutil import launch_override, assert_close, log, sample_rows, to_dev, to_np, torch_dtype
from test_gpu_attn import GpuStream, _swk
from test_gpu_recache import _read_frame

pytestmark = pytest.mark.gpu


def _weights_dev(ws, dtype):
    """[C, H*D] oracle orientation -> [H*D, C] device tensors ([out, in] layout)."""
    return [to_dev(np.ascontiguousarray(w.T), dtype) for w in ws]


def _project_stream(w, chunks, tile=None, eps=None, check_rows=None, attend=True):
    """Stream `chunks` through sa_cache_project_append and the oracle; check q, the cache and attention."""
    import torch
    swk = _swk()
    gs = GpuStream(w, eps=eps)
    wq, wk, wv = wl.projection_weights(w)
    dq, dk, dv = _weights_dev((wq, wk, wv), w.dtype)
    T = w.tokens_per_frame
    f0, t0 = 0, 0
    with launch_override(tile=tile):
        for c in chunks:
            x = wl.frame_hidden(w, f0, c)
            q_out = torch.empty((w.batch, c * T, w.n_heads, w.head_dim), dtype=torch_dtype(w.dtype), device="cuda")
            swk.sa_cache_project_append(gs.cache, to_dev(x, w.dtype), dq, dk, dv, w.hidden, q_out, c, t0)
            torch.cuda.synchronize()
            q_ref, _ = oproject.project_append(gs.oracle, x, wq, wk, wv, w.n_heads, t0)
            rows = check_rows(c * T) if check_rows else slice(None)
            assert_close(to_np(q_out)[:, rows], q_ref[:, rows], w.dtype, f"q of frames {f0}..{f0 + c - 1}")
            assert [(s.frame, s.t, s.segment, s.slot) for s in swk.sa_cache_slots(gs.cache)] == \
                [(s.frame, s.t, s.segment, s.slot) for s in gs.oracle.model.slots()]
            res = gs.oracle.resident()
            for j in range(c):   # the chunk's own frames, as stored
                idx = len(res) - c + j
                ko, vo = _read_frame(gs, idx)
                kref, vref = gs.oracle.frame_kv(res[idx])
                fr = check_rows(T) if check_rows else slice(None)
                assert_close(to_np(ko)[:, fr], kref[:, fr], w.dtype, f"K of frame {res[idx]}")
                assert_close(to_np(vo)[:, fr], vref[:, fr], w.dtype, f"V of frame {res[idx]}")
            if attend:
                # attention on the projected queries; the oracle attends with its own fp64 q
                o = torch.empty_like(q_out)
                nbytes = swk.sa_window_attn_workspace(gs.cache, c)
                ws = torch.zeros(max(nbytes // 4, 4), dtype=torch.float32, device="cuda")
                swk.sa_window_attn(gs.cache, q_out, o, c, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws)
                torch.cuda.synchronize()
                arows = check_rows(c * T) if check_rows else None
                ref = gs.oracle.attend(q_ref, causal=True, rows=arows)
                got = to_np(o) if arows is None else to_np(o)[:, arows]
                rel, mx = assert_close(got, ref, w.dtype, f"attention of frames {f0}..{f0 + c - 1}")
                log(f"  chunk at frame {f0}: attention rel_l2 {rel:.2e} max_abs {mx:.2e}")
            f0 += c
            t0 += c
    return gs


SMALL = wl.Workload("project-small", 46, batch=2, n_heads=4, head_dim=128, dims=(44, 42, 42), grid=(4, 10),
                    n_sink=2, n_local=3, chunk=1, frames=8, dtype="bf16", sigma=0.8, hidden=256)


@pytest.mark.parametrize("tile", [None, "0", "1", "2", "3"])
def test_project_append_stream_small(tile):
    """Chunks of 1-3 frames through sinks, ring wrap and eviction; every tile shape of the GEMM."""
    _project_stream(SMALL, [1, 2, 1, 3, 1, 2], tile=tile, eps=wl.head_jitter(SMALL))


def test_project_append_ragged_d64():
    """head_dim 64, 3 heads (q, k, v segments of 192 features straddle 128/256-feature tiles), hidden 96."""
    w = wl.Workload("project-d64", 47, batch=3, n_heads=3, head_dim=64, dims=(22, 22, 20), grid=(6, 12),
                    n_sink=1, n_local=2, chunk=1, frames=5, dtype="bf16", hidden=96)
    for tile in ("0", "1", "2", "3"):
        log(f"d64 tile {tile}")
        _project_stream(w, [1, 1, 2, 1], tile=tile)


def test_project_append_f32():
    w = wl.Workload("project-f32", 48, batch=1, n_heads=2, head_dim=64, dims=(22, 22, 20), grid=(8, 8),
                    n_sink=1, n_local=2, chunk=1, frames=5, dtype="f32", hidden=128)
    _project_stream(w, [1, 1, 2, 1])


def test_project_append_wan_layer():
    """Wan-1.3B layer (hidden 1536, 12 x 128 heads, 30 x 52 grid, 3 sink + 9 local): 13 single frames,
    sampled rows of q, K, V and attention checked on every frame."""
    w = wl.Workload("project-wan13b", 49, batch=1, n_heads=12, head_dim=128, dims=(44, 42, 42), grid=(30, 52),
                    n_sink=3, n_local=9, chunk=1, frames=13, dtype="bf16", hidden=1536)
    rows = lambda L: sample_rows(L, 1560, n=96, seed=L)  # noqa: E731
    _project_stream(w, [1] * 13, check_rows=rows)


def test_project_append_without_q_and_errors():
    """w_q = q_out = NULL writes only the cache; rejected calls leave the cache unchanged."""
    import torch
    swk = _swk()
    w = SMALL
    gs = GpuStream(w)
    wq, wk, wv = wl.projection_weights(w)
    dq, dk, dv = _weights_dev((wq, wk, wv), w.dtype)
    T = w.tokens_per_frame
    x = wl.frame_hidden(w, 0, 1)
    tx = to_dev(x, w.dtype)
    swk.sa_cache_project_append(gs.cache, tx, None, dk, dv, w.hidden, None, 1, 0)
    torch.cuda.synchronize()
    q, _ = oproject.project_append(gs.oracle, x, None, wk, wv, w.n_heads, 0)
    assert q is None
    ko, vo = _read_frame(gs, 0)
    kref, vref = gs.oracle.frame_kv(0)
    assert_close(to_np(ko), kref, w.dtype, "K without q")
    assert_close(to_np(vo), vref, w.dtype, "V without q")
    q_out = torch.empty((w.batch, T, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    before = swk.sa_cache_counts(gs.cache)
    cases = [
        (dict(w_q=dq, q_out=None), swk.SA_ERR_NULL),          # q weights without an output
        (dict(t0=0), swk.SA_ERR_RANGE),                        # time not after the newest
        (dict(n_frames=5), swk.SA_ERR_RANGE),                  # 4 non-sink frames > the 3-frame ring
        (dict(hidden=48), swk.SA_ERR_SHAPE),                   # not a multiple of 32
    ]
    for kw, status in cases:
        args = dict(w_q=dq, q_out=q_out, hidden=w.hidden, n_frames=1, t0=5)
        args.update(kw)
        with pytest.raises(swk.SinkAttnError) as ei:
            swk.sa_cache_project_append(gs.cache, tx, args["w_q"], dk, dv, args["hidden"], args["q_out"],
                                        args["n_frames"], args["t0"])
        assert ei.value.status == status, kw
        assert swk.sa_cache_counts(gs.cache) == before


def test_cache_calls_reject_buffers_on_the_stores():
    """Inputs and outputs placed on the cache's own stores (or q_out on x) are SA_ERR_RANGE, cache unchanged."""
    import torch
    swk = _swk()
    w = SMALL
    gs = GpuStream(w, with_oracle=False)
    wq, wk, wv = wl.projection_weights(w)
    dq, dk, dv = _weights_dev((wq, wk, wv), w.dtype)
    T = w.tokens_per_frame
    shape = (w.batch, T, w.n_heads, w.head_dim)
    n = w.batch * T * w.n_heads * w.head_dim
    tx = to_dev(wl.frame_hidden(w, 0, 1), w.dtype)
    swk.sa_cache_project_append(gs.cache, tx, None, dk, dv, w.hidden, None, 1, 0)
    torch.cuda.synchronize()
    before = swk.sa_cache_counts(gs.cache)
    ks, vs = gs.cache.k_store, gs.cache.v_store
    z = torch.zeros(shape, dtype=ks.dtype, device="cuda")
    nx = tx.numel()
    buf = torch.zeros(nx + n, dtype=tx.dtype, device="cuda")
    x2 = buf[:nx].view(tx.shape)
    x2.copy_(tx)
    q_on_x = buf[nx // 2:nx // 2 + n].view(shape)
    calls = [
        lambda: swk.sa_cache_append(gs.cache, ks[:n].view(shape), z, 1, 1),                   # k on the key store
        lambda: swk.sa_cache_append(gs.cache, z, vs[n:2 * n].view(shape), 1, 1),              # v on the value store
        lambda: swk.sa_cache_read(gs.cache, 0, k_out=vs[:n].view(shape)),                     # read into a store
        lambda: swk.sa_cache_recache(gs.cache, ks[:nx].view(tx.shape), dk, dv, w.hidden),     # x on the key store
        lambda: swk.sa_cache_project_append(gs.cache, tx, None, dk, vs[:dv.numel()].view(dv.shape), w.hidden, None,
                                            1, 1),                                           # w_v on the value store
        lambda: swk.sa_cache_project_append(gs.cache, x2, dq, dk, dv, w.hidden, q_on_x, 1, 1),  # q_out on x
    ]
    for i, call in enumerate(calls):
        with pytest.raises(swk.SinkAttnError) as ei:
            call()
        assert ei.value.status == swk.SA_ERR_RANGE, i
        assert swk.sa_cache_counts(gs.cache) == before, i


@pytest.mark.parametrize("n_rows,fin,fout,dtype", [
    (1560, 1536, 1536, "bf16"),   # the output projection of one Wan-1.3B frame
    (333, 96, 80, "bf16"),        # ragged rows, 80 outputs (padding in every tile shape)
    (4680, 1536, 1536, "bf16"),   # a 3-frame chunk
    (77, 64, 48, "f32"),
])
def test_linear(n_rows, fin, fout, dtype):
    import torch
    swk = _swk()
    w = wl.Workload("linear", 50, batch=1, n_heads=1, head_dim=fin, dims=(0, 0, 0), grid=(1, 1),
                    n_sink=0, n_local=1, chunk=1, frames=1, dtype=dtype, hidden=fout)
    x = wl.normal((n_rows, fin), 50, 0, 0, 0, wl.TENSOR_X, 1.0, dtype)
    wo = wl.output_weight(w)          # [fin, fout]
    ref = oproject.linear(x, wo)
    tx = to_dev(x, dtype)
    tw = to_dev(np.ascontiguousarray(wo.T), dtype)
    for tile in ((None, "0", "1", "2", "3") if dtype == "bf16" else (None,)):
        y = torch.full((n_rows, fout), float("nan"), dtype=torch_dtype(dtype), device="cuda")
        with launch_override(tile=tile):
            swk.sa_linear(tx, tw, y, n_rows, fin, fout)
        torch.cuda.synchronize()
        rel, mx = assert_close(to_np(y), ref, dtype, f"linear {n_rows}x{fin}->{fout} tile {tile}")
        log(f"  linear {n_rows}x{fin}->{fout} tile {tile}: rel_l2 {rel:.2e} max_abs {mx:.2e}")
    # library cross-check on the device (fp32 matmul of the same values)
    yt = (tx.float() @ tw.float().t())
    assert (y.float() - yt).abs().max().item() <= (2e-2 if dtype == "bf16" else 1e-4)
    # zero rows: nothing launched, nothing written
    swk.sa_linear(tx, tw, y, 0, fin, fout)
