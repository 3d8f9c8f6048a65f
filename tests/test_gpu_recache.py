"""GPU parity: sa_cache_recache (KV recache at a prompt switch) vs the fp64 oracle."""
import numpy as np
import pytest

import workloads as wl
from oracle import recache as orecache
from swk_testutil import launch_override, assert_close, log, sample_rows, to_dev, to_np, torch_dtype
from test_gpu_attn import GpuStream, _check, _swk

pytestmark = pytest.mark.gpu


def _read_frame(gs, idx):
    import torch
    w = gs.w
    shape = (w.batch, w.tokens_per_frame, w.n_heads, w.head_dim)
    ko = torch.empty(shape, dtype=torch_dtype(w.dtype), device="cuda")
    vo = torch.empty_like(ko)
    _swk().sa_cache_read(gs.cache, idx, ko, vo)
    torch.cuda.synchronize()
    return ko, vo


def test_cfg4_prompt_switch_recache_stream():
    """30 frames, recache (x [18720 x 1536], fresh W) after frame 29, then 30 more frames."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[4]
    gs = GpuStream(w)
    T = w.tokens_per_frame
    rows = sample_rows(T, T, n=80, seed=2)
    for f in range(w.recache_after):
        k = wl.frame_qkv(w, f, tensor=wl.TENSOR_K)
        v = wl.frame_qkv(w, f, tensor=wl.TENSOR_V)
        gs.append(k, v, 1, f)
    x, wk, wv = wl.recache_inputs(w)
    log("cfg4 recache")
    wk_t = to_dev(np.ascontiguousarray(wk.T), "bf16")  # [H*D, C] (out, in)
    wv_t = to_dev(np.ascontiguousarray(wv.T), "bf16")
    tx = to_dev(x, "bf16")
    slots_before = [(s.frame, s.t, s.segment, s.slot) for s in swk.sa_cache_slots(gs.cache)]
    swk.sa_cache_recache(gs.cache, tx, wk_t, wv_t, w.hidden)
    torch.cuda.synchronize()
    gs.oracle.recache(x, wk, wv)
    assert [(s.frame, s.t, s.segment, s.slot) for s in swk.sa_cache_slots(gs.cache)] == slots_before
    res = gs.oracle.resident()
    for idx in (0, 2, 3, len(res) - 1):
        ko, vo = _read_frame(gs, idx)
        kref, vref = gs.oracle.frame_kv(res[idx])
        assert_close(to_np(ko), kref, "bf16", f"recached K frame {res[idx]}")
        assert_close(to_np(vo), vref, "bf16", f"recached V frame {res[idx]}")
    # library cross-check on the device: V of the last frame vs torch.matmul (bf16 in, fp32 accumulate)
    xl = tx[0, (len(res) - 1) * T:len(res) * T].float()
    vt = (xl @ wv_t.float().t()).reshape(T, w.n_heads, w.head_dim)
    _, vo = _read_frame(gs, len(res) - 1)
    diff = (vo[0].float() - vt).abs().max().item()
    assert diff <= 2e-2, f"recache V vs torch.matmul: {diff}"
    for f in range(w.recache_after, w.frames):
        q = wl.frame_qkv(w, f, tensor=wl.TENSOR_Q)
        k = wl.frame_qkv(w, f, tensor=wl.TENSOR_K)
        v = wl.frame_qkv(w, f, tensor=wl.TENSOR_V)
        gs.append(k, v, 1, f)
        if f in (30, 31, 38, 39):
            o = gs.attend(q, 1, swk.SA_MASK_FRAME_CAUSAL)
            _check(gs, q, o, True, rows=rows, what=f"cfg4 frame {f} after recache")


def test_recache_idempotent_bit_exact_and_matches_append():
    """Recache twice with the same W -> identical bits; recache from x equals appending x.W (within tol)."""
    import torch
    swk = _swk()
    w = wl.Workload("recache-small", 43, batch=2, n_heads=4, head_dim=128, dims=(44, 42, 42), grid=(4, 10),
                    n_sink=2, n_local=3, chunk=1, frames=7, dtype="bf16", sigma=0.8, hidden=256)
    eps = wl.head_jitter(w)
    gs = GpuStream(w, eps=eps)
    T = w.tokens_per_frame
    x, wk, wv = wl.recache_inputs(w, n_frames=w.frames)
    # fill by appending K = x.W_k, V = x.W_v (computed in fp64, rounded to bf16)
    for f in range(w.frames):
        xs = x[:, f * T:(f + 1) * T]
        k = wl.to_bf16_values(orecache.project(xs, wk, w.n_heads).astype(np.float32))
        v = wl.to_bf16_values(orecache.project(xs, wv, w.n_heads).astype(np.float32))
        gs.append(k, v, 1, 5 + f)
    res = gs.oracle.resident()
    xr = np.concatenate([x[:, f * T:(f + 1) * T] for f in res], axis=1)
    tx = to_dev(xr, "bf16")
    wk_t = to_dev(np.ascontiguousarray(wk.T), "bf16")
    wv_t = to_dev(np.ascontiguousarray(wv.T), "bf16")
    swk.sa_cache_recache(gs.cache, tx, wk_t, wv_t, w.hidden)
    first = [_read_frame(gs, i) for i in range(len(res))]
    swk.sa_cache_recache(gs.cache, tx, wk_t, wv_t, w.hidden)
    second = [_read_frame(gs, i) for i in range(len(res))]
    for (k1, v1), (k2, v2) in zip(first, second):
        assert torch.equal(k1, k2) and torch.equal(v1, v2)
    appended = {f: gs.oracle.frame_kv(f) for f in res}   # RoPE(bf16(x.W_k)) and bf16(x.W_v)
    gs.oracle.recache(xr, wk, wv)                          # exact fp64 recache
    for i, f in enumerate(res):
        kref, vref = gs.oracle.frame_kv(f)
        assert_close(to_np(first[i][0]), kref, "bf16", f"recache K frame {f}")
        assert_close(to_np(first[i][1]), vref, "bf16", f"recache V frame {f}")
        # same cache as appending x.W: the two paths round to bf16 at different
        # points (after vs before the rotation), so each rotated pair agrees to
        # about one bf16 ulp of the pair's norm (|k| reaches ~5 here, so the
        # 2e-2 absolute bound of the attention outputs does not apply)
        for got, ref in ((first[i][0], appended[f][0]), (first[i][1], appended[f][1])):
            g = to_np(got).reshape(-1, 2)
            r = ref.reshape(-1, 2)
            err = np.linalg.norm(g - r, axis=1)
            assert np.all(err <= 2.0 ** -7 * np.linalg.norm(r, axis=1) + 1e-6), f"frame {f}: {err.max()}"


def test_recache_f32_small():
    import torch
    swk = _swk()
    w = wl.Workload("recache-f32", 44, batch=1, n_heads=2, head_dim=64, dims=(22, 22, 20), grid=(8, 8),
                    n_sink=1, n_local=2, chunk=1, frames=5, dtype="f32", hidden=128)
    gs = GpuStream(w)
    for f in range(w.frames):
        gs.append(wl.frame_qkv(w, f, tensor=wl.TENSOR_K), wl.frame_qkv(w, f, tensor=wl.TENSOR_V), 1, f)
    res = gs.oracle.resident()
    x, wk, wv = wl.recache_inputs(w, n_frames=len(res))
    swk.sa_cache_recache(gs.cache, to_dev(x, "f32"), to_dev(np.ascontiguousarray(wk.T), "f32"),
                         to_dev(np.ascontiguousarray(wv.T), "f32"), w.hidden)
    torch.cuda.synchronize()
    gs.oracle.recache(x, wk, wv)
    for i, f in enumerate(res):
        ko, vo = _read_frame(gs, i)
        kref, vref = gs.oracle.frame_kv(f)
        assert_close(to_np(ko), kref, "f32", f"f32 recache K frame {f}")
        assert_close(to_np(vo), vref, "f32", f"f32 recache V frame {f}")
    q = wl.frame_qkv(w, 4, tensor=wl.TENSOR_Q)
    o = gs.attend(q, 1, swk.SA_MASK_FRAME_CAUSAL)
    _check(gs, q, o, True, what="f32 attention after recache")


def test_recache_errors():
    import torch
    swk = _swk()
    w = wl.WORKLOADS[1]
    gs = GpuStream(w, with_oracle=False)
    x = torch.zeros((1, 3 * w.tokens_per_frame, 64), device="cuda")
    wk = torch.zeros((w.n_heads * w.head_dim, 64), device="cuda")
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_recache(gs.cache, x, wk, wk, 64)
    assert e.value.status == swk.SA_ERR_STATE
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_recache(gs.cache, x, wk, wk, 60)
    assert e.value.status == swk.SA_ERR_SHAPE


@pytest.mark.parametrize("n_heads,head_dim,dims,grid,hidden", [
    # 2*H*D = 384: the K/V boundary (192) falls inside the first 256-feature
    # tile and the second tile is half padding; 576 tokens = 4.5 token tiles;
    # hidden 192 = 6 reduction slices
    (3, 64, (22, 22, 20), (6, 12), 192),
    # 2*H*D = 640 (2.5 feature tiles, boundary at 320 inside the second);
    # tokens per frame 40 so 128-token tiles cross frames and streams
    (5, 64, (22, 22, 20), (4, 10), 320),
])
@pytest.mark.parametrize("tile", [None, "3"])
def test_recache_bf16_ragged_tiles(n_heads, head_dim, dims, grid, hidden, tile):
    """bf16 recache where features and tokens do not fill whole GEMM tiles, with a wrapped ring; the automatic
    tile and the 256 x 256 eight-wave tile."""
    import torch
    swk = _swk()
    w = wl.Workload("recache-ragged", 45, batch=2, n_heads=n_heads, head_dim=head_dim, dims=dims, grid=grid,
                    n_sink=1, n_local=3, chunk=1, frames=7, dtype="bf16", sigma=0.8, hidden=hidden)
    eps = wl.head_jitter(w)
    gs = GpuStream(w, eps=eps)
    for f in range(w.frames):
        gs.append(wl.frame_qkv(w, f, tensor=wl.TENSOR_K), wl.frame_qkv(w, f, tensor=wl.TENSOR_V), 1, f)
    res = gs.oracle.resident()
    x, wk, wv = wl.recache_inputs(w, n_frames=len(res))
    log(f"recache ragged H={n_heads} D={head_dim} grid={grid} hidden={hidden} resident={res}")
    with launch_override(tile=tile):
        swk.sa_cache_recache(gs.cache, to_dev(x, "bf16"), to_dev(np.ascontiguousarray(wk.T), "bf16"),
                             to_dev(np.ascontiguousarray(wv.T), "bf16"), w.hidden)
    torch.cuda.synchronize()
    gs.oracle.recache(x, wk, wv)
    for i, f in enumerate(res):
        ko, vo = _read_frame(gs, i)
        kref, vref = gs.oracle.frame_kv(f)
        assert_close(to_np(ko), kref, "bf16", f"ragged recache K frame {f}")
        assert_close(to_np(vo), vref, "bf16", f"ragged recache V frame {f}")
    q = wl.frame_qkv(w, w.frames - 1, tensor=wl.TENSOR_Q)
    o = gs.attend(q, 1, swk.SA_MASK_FRAME_CAUSAL)
    _check(gs, q, o, True, what="attention after ragged recache")
