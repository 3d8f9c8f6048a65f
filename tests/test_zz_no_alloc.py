"""GPU: sa_window_attn_noalloc (key-split partials in the library's own device scratch) against
sa_window_attn with a caller workspace, through the C-ABI, on two calls in a row -- the second with a
smaller input -- and the size limit.  Both paths run the same kernels, so the outputs must be
bit-identical (a stronger bar than the bf16 tolerance)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl
from swk_testutil import launch_override, log, to_dev

pytestmark = pytest.mark.gpu


def _swk():
    import sink_window_kv_amd as swk
    return swk


def _filled_cache(w, n_frames, seed_layer):
    swk = _swk()
    eps = wl.head_jitter(w, layer=seed_layer) if w.sigma > 0 else None
    rope = swk.Rope(w.n_heads, w.head_dim, w.dims, w.grid, w.theta0, w.sigma, eps)
    cache = swk.Cache(rope, w.batch, w.n_sink, w.n_local, torch.bfloat16)
    for f in range(n_frames):
        k, v = (wl.frame_qkv(w, f, layer=seed_layer, tensor=t) for t in (wl.TENSOR_K, wl.TENSOR_V))
        swk.sa_cache_append(cache, to_dev(k, "bf16"), to_dev(v, "bf16"), 1, f)
    return rope, cache


def _both(cache, q, n_q, mask, scale=0.0):
    swk = _swk()
    nbytes = swk.sa_window_attn_workspace(cache, n_q)
    ws = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device="cuda")
    o_ref = torch.empty_like(q)
    o_na = torch.full_like(q, float("nan"))
    swk.sa_window_attn(cache, q, o_ref, n_q, scale, mask, ws)
    swk.sa_window_attn_noalloc(cache, q, o_na, n_q, scale, mask)
    torch.cuda.synchronize()
    return nbytes, o_ref, o_na


@pytest.mark.parametrize("kernel", [None, "3"])
def test_noalloc_matches_workspace_entry_point_two_calls(kernel):
    """The default attention kernel, and the 64-row pipelined variant (its O accumulators in AGPRs)."""
    swk = _swk()
    # call 1: the Wan-1.3B layer in steady state (1560 queries over 12 frames, 3 key splits: 29.2 MB of partials)
    w1 = wl.WORKLOADS[2]
    log(f"noalloc call 1: Wan-1.3B layer, frame 13, kernel {kernel}")
    rope1, c1 = _filled_cache(w1, 14, 0)
    q1 = to_dev(wl.frame_qkv(w1, 13, tensor=wl.TENSOR_Q, scale=1.0), "bf16")
    with launch_override(kernel=kernel):
        n1, ref1, got1 = _both(c1, q1, 1, swk.SA_MASK_FRAME_CAUSAL)
    assert n1 > 0, "the first call must use the scratch (key splits)"
    assert torch.equal(got1, ref1), "call 1: noalloc output differs from sa_window_attn"
    # call 2: smaller (2 heads, 200 tokens per frame, a 2-frame frame-causal chunk, 5 forced key splits)
    w2 = dataclasses.replace(wl.WORKLOADS[3], name="noalloc-small", n_heads=2, grid=(10, 20), n_sink=1,
                             n_local=4, sigma=0.8)
    log(f"noalloc call 2: H=2, T=200, 2-frame chunk, 5 splits, kernel {kernel}")
    with launch_override(kernel=kernel, splits=5):
        rope2, c2 = _filled_cache(w2, 7, 1)
        q2 = to_dev(np.concatenate([wl.frame_qkv(w2, f, layer=1, tensor=wl.TENSOR_Q, scale=1.0)
                                    for f in (5, 6)], axis=1), "bf16")
        n2, ref2, got2 = _both(c2, q2, 2, swk.SA_MASK_FRAME_CAUSAL, scale=0.3)
    assert 0 < n2 < n1
    assert torch.equal(got2, ref2), "call 2: noalloc output differs from sa_window_attn"
    assert torch.isfinite(got2.float()).all()
    # the first cache again after the smaller call (the scratch keeps the last call's bytes)
    o_again = torch.empty_like(q1)
    with launch_override(kernel=kernel):
        swk.sa_window_attn_noalloc(c1, q1, o_again, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(o_again, ref1)
    for c, r in ((c1, rope1), (c2, rope2)):
        c.close()
        r.close()


def test_noalloc_rejects_partials_beyond_its_scratch():
    swk = _swk()
    w = wl.WORKLOADS[2]
    rope, cache = _filled_cache(w, 12, 0)
    q = to_dev(wl.frame_qkv(w, 11, tensor=wl.TENSOR_Q), "bf16")
    o = torch.zeros_like(q)
    with launch_override(splits=5):          # 5 x 18720 rows x 130 x 4 B = 48.7 MB > 32 MiB
        assert swk.sa_window_attn_workspace(cache, 1) > 32 << 20
        with pytest.raises(swk.SinkAttnError) as e:
            swk.sa_window_attn_noalloc(cache, q, o, 1)
    assert e.value.status == swk.SA_ERR_RANGE
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(o)) == 0
    cache.close()
    rope.close()
