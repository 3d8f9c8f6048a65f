"""GPU parity: sa_window_attn_sink_mass (softmax mass on the sink frames per row and head) vs the fp64 oracle."""
import numpy as np
import pytest

import workloads as wl
from oracle import diagnostics as odiag
from swk_testutil import launch_override, assert_close, log, sample_rows, to_dev, to_np
from test_gpu_attn import GpuStream, _swk

pytestmark = pytest.mark.gpu


def _mass_call(gs, q, n_q, mask, scale=0.0):
    """Run sa_window_attn_sink_mass and plain sa_window_attn on the same inputs; o must be bit-identical."""
    import torch
    swk = _swk()
    tq = to_dev(q, gs.w.dtype)
    B, Lq, H = q.shape[0], q.shape[1], q.shape[2]
    nbytes = swk.sa_window_attn_workspace(gs.cache, n_q)
    ws = torch.zeros(max(nbytes // 4, 4), dtype=torch.float32, device="cuda")
    o1 = torch.empty_like(tq)
    mass = torch.full((B, Lq, H), float("nan"), dtype=torch.float32, device="cuda")
    swk.sa_window_attn_sink_mass(gs.cache, tq, o1, mass, n_q, scale, mask, ws)
    o2 = torch.empty_like(tq)
    swk.sa_window_attn(gs.cache, tq, o2, n_q, scale, mask, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "attention output differs from sa_window_attn"
    return to_np(mass)


def _check_mass(gs, q, n_q, mask, rows=None, what="", scale=0.0):
    swk = _swk()
    got = _mass_call(gs, q, n_q, mask, scale)
    ref = odiag.sink_mass(gs.oracle, q, mask == swk.SA_MASK_FRAME_CAUSAL, scale=scale or None, rows=rows)
    if rows is not None:
        got = got[:, rows]
    rel, mx = assert_close(got, ref, gs.w.dtype, what)
    log(f"  {what}: mass mean {ref.mean():.3f} rel_l2 {rel:.2e} max_abs {mx:.2e}")


SMALL = wl.Workload("mass-small", 51, batch=2, n_heads=4, head_dim=128, dims=(44, 42, 42), grid=(4, 10),
                    n_sink=2, n_local=3, chunk=1, frames=8, dtype="bf16", sigma=0.8)


@pytest.mark.parametrize("kernel", ["1", "2", "3"])
def test_sink_mass_small_stream(kernel):
    """Every frame from the first (query frames that are sinks: mass 1) through eviction; both masks;
    unscaled N(0,1) queries and keys so the softmax is sharp and the mass varies."""
    swk = _swk()
    w = SMALL
    gs = GpuStream(w, eps=wl.head_jitter(w))
    with launch_override(kernel=kernel):
        for f in range(w.frames):
            q, k, v = (wl.frame_qkv(w, f, tensor=t, scale=1.0) for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
            gs.append(k, v, 1, f)
            for mask in (swk.SA_MASK_NONE, swk.SA_MASK_FRAME_CAUSAL):
                _check_mass(gs, q, 1, mask, what=f"frame {f} mask {mask}")


def test_sink_mass_chunks_b2():
    """3-frame chunks, frame-causal (query frames see different numbers of frames), 2 streams."""
    swk = _swk()
    w = wl.Workload("mass-chunk", 52, batch=2, n_heads=3, head_dim=64, dims=(22, 22, 20), grid=(6, 12),
                    n_sink=3, n_local=6, chunk=3, frames=15, dtype="bf16", sigma=0.8)
    gs = GpuStream(w, eps=wl.head_jitter(w))
    for f0 in range(0, w.frames, 3):
        q, k, v = (wl.chunk_qkv(w, f0, 3, tensor=t, scale=1.0) for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
        gs.append(k, v, 3, f0)
        _check_mass(gs, q, 3, swk.SA_MASK_FRAME_CAUSAL, what=f"chunk at {f0}")


@pytest.mark.parametrize("splits,kernel", [(None, None), ("1", None), ("5", None), (None, "2"), (None, "3")])
def test_sink_mass_wan_layer(splits, kernel):
    """Wan-1.3B layer in steady state (3 sinks + 9 local, 18720 keys), sampled rows, all heads,
    LoL jitter sigma = 0.8; launch shapes forced as for the attention."""
    swk = _swk()
    w = wl.WORKLOADS[3]
    gs = GpuStream(w, eps=wl.head_jitter(w))
    T = w.tokens_per_frame
    rows = sample_rows(T, T, n=64, seed=7)
    with launch_override(splits=splits, kernel=kernel):
        for f in range(14):
            gs.append(wl.frame_qkv(w, f, tensor=wl.TENSOR_K), wl.frame_qkv(w, f, tensor=wl.TENSOR_V), 1, f)
            if f in (0, 2, 5, 13):
                for scale in (None, 1.0):
                    q = wl.frame_qkv(w, f, tensor=wl.TENSOR_Q, scale=scale)
                    _check_mass(gs, q, 1, swk.SA_MASK_FRAME_CAUSAL, rows=rows, what=f"wan frame {f} q scale {scale}")


def test_sink_mass_f32_and_no_sinks():
    """fp32 path at 1e-5; a cache without sinks gives mass 0 and the plain attention output."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[1]
    gs = GpuStream(w)
    for f in range(w.frames):
        q, k, v = (wl.frame_qkv(w, f, tensor=t) for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
        gs.append(k, v, 1, f)
        for mask in (swk.SA_MASK_NONE, swk.SA_MASK_FRAME_CAUSAL):
            _check_mass(gs, q, 1, mask, what=f"f32 frame {f} mask {mask}")
    w0 = wl.Workload("mass-nosink", 53, batch=1, n_heads=2, head_dim=128, dims=(44, 42, 42), grid=(4, 8),
                     n_sink=0, n_local=3, chunk=1, frames=5, dtype="bf16")
    gs0 = GpuStream(w0)
    for f in range(w0.frames):
        q, k, v = (wl.frame_qkv(w0, f, tensor=t) for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
        gs0.append(k, v, 1, f)
        assert np.all(_mass_call(gs0, q, 1, swk.SA_MASK_FRAME_CAUSAL) == 0.0)
    # argument checks
    q = to_dev(wl.frame_qkv(w0, 4, tensor=wl.TENSOR_Q), "bf16")
    o = torch.empty_like(q)
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_window_attn_sink_mass(gs0.cache, q, o, None, 1)
    assert e.value.status == swk.SA_ERR_NULL
    rows = q.shape[1] * q.shape[2]
    for target in (o, q, gs0.cache.k_store):          # sink_mass placed on another buffer
        with pytest.raises(swk.SinkAttnError) as e:
            swk.sa_window_attn_sink_mass(gs0.cache, q, o, target.view(-1)[:2 * rows].view(torch.float32), 1)
        assert e.value.status == swk.SA_ERR_RANGE
