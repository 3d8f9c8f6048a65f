"""GPU parity: the 8-bit projections (sa_quantize_rows, sa_linear_q8, sa_cache_recache_q8,
sa_cache_project_append_q8) vs the oracle.

The codes and scales the GEMM tests upload come from the oracle's quantisation;
sa_quantize_rows is checked against it separately (bit-exact).  int8 outputs
are bit-exact (integer sums, the same fp32 scaling steps, bf16 rounding);
e4m3 outputs and everything rotated are held to the bf16 tolerances.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import project as oproject
from oracle import quant as oquant
from swk_testutil import launch_override, assert_close, log, sample_rows, to_dev, to_np, torch_dtype
from test_gpu_attn import GpuStream, _check, _swk
from test_gpu_recache import _read_frame

pytestmark = pytest.mark.gpu

QTYPES = ["int8", "e4m3"]


def _qcode(name):
    return _swk().SA_Q_INT8 if name == "int8" else _swk().SA_Q_E4M3


def _bytes_dev(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8).copy()).cuda()


def _f32_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy()).cuda()


def _bf16_bits(x):
    """bf16 (nearest even) bit patterns of float32 values, via torch's conversion on the host."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy()


def _quantize(x2d, qtype):
    """Oracle codes and scales of the rows of x2d, plus their device copies."""
    c, s = oquant.quantize_rows(x2d, qtype)
    return c, s, _bytes_dev(c), _f32_dev(s)


def _spread_rows(n, C, seed):
    """bf16 rows with magnitudes from 2^-12 to 2^12, a zero row and a row with one nonzero value."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, C)).astype(np.float32) * np.exp2(g.integers(-12, 13, size=(n, 1))).astype(np.float32)
    x[min(3, n - 1)] = 0.0
    if n > 5:
        x[5] = 0.0
        x[5, C // 3] = -1.75
    return wl.to_bf16_values(x)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("n,C", [(1563, 1536), (37, 64), (6, 4616)])
def test_quantize_rows_bit_exact(qtype, n, C):
    """Codes and scales equal the oracle's fp32 decisions bit for bit."""
    import torch
    swk = _swk()
    x = _spread_rows(n, C, seed=C + n)
    log(f"quantize {qtype} {n}x{C}")
    codes = torch.empty((n, C), dtype=torch.uint8, device="cuda")
    scales = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    swk.sa_quantize_rows(to_dev(x, "bf16"), codes, scales, _qcode(qtype))
    torch.cuda.synchronize()
    c_ref, s_ref = oquant.quantize_rows(x, qtype)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    got = codes.cpu().numpy()
    ref = c_ref.view(np.uint8)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"


def _linear_case(n, C, F, qtype, tile, seed):
    import torch
    swk = _swk()
    g = np.random.default_rng(seed)
    x = wl.to_bf16_values(g.standard_normal((n, C)).astype(np.float32))
    w = wl.to_bf16_values((g.standard_normal((F, C)) / np.sqrt(C)).astype(np.float32))
    cx, sx, dcx, dsx = _quantize(x, qtype)
    cw, sw, dcw, dsw = _quantize(w, qtype)
    y = torch.empty((n, F), dtype=torch.bfloat16, device="cuda")
    with launch_override(tile=tile):
        swk.sa_linear_q8(dcx, dsx, dcw, dsw, y, _qcode(qtype), n, C, F)
    torch.cuda.synchronize()
    ref = oquant.linear_q8(cx, sx, cw, sw, qtype)
    if qtype == "int8":
        got = y.view(torch.int16).cpu().numpy()
        want = _bf16_bits(ref)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} of {got.size} outputs differ, first at {bad[:3].tolist()}"
    else:
        rel, mx = assert_close(to_np(y), ref, "bf16", f"linear_q8 e4m3 {n}x{C}->{F}")
        log(f"  e4m3 {n}x{C}->{F} tile {tile}: rel_l2 {rel:.2e} max_abs {mx:.2e}")
    return y


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("tile", [None, "0", "1", "2", "3"])
def test_linear_q8_output_projection_shape(qtype, tile):
    """One frame's output projection (1560 x 1536 -> 1536) in every tile shape; int8 bit-exact."""
    log(f"linear_q8 {qtype} tile {tile}")
    _linear_case(1560, 1536, 1536, qtype, tile, seed=11)


@pytest.mark.parametrize("qtype", QTYPES)
def test_linear_q8_ragged(qtype):
    """Ragged rows and features (partial token and feature tiles), short and long reductions."""
    for (n, C, F) in [(100, 128, 48), (1, 64, 16), (257, 1024, 272), (70, 4608, 64)]:
        for tile in ("0", "1", "2"):
            log(f"linear_q8 {qtype} {n}x{C}->{F} tile {tile}")
            _linear_case(n, C, F, qtype, tile, seed=n + C + F)


@pytest.mark.parametrize("qtype", QTYPES)
def test_recache_q8_prompt_switch(qtype):
    """Wan-1.3B layer: 30 frames, an 8-bit recache (x [18720 x 1536] per token, W per output feature) after
    frame 29, then frames 30-31: recached K/V and the attention vs the oracle on the dequantized operands."""
    import torch
    swk = _swk()
    w = wl.WORKLOADS[4]
    gs = GpuStream(w)
    T = w.tokens_per_frame
    for f in range(w.recache_after):
        gs.append(wl.frame_qkv(w, f, tensor=wl.TENSOR_K), wl.frame_qkv(w, f, tensor=wl.TENSOR_V), 1, f)
    x, wk, wv = wl.recache_inputs(w)
    C = w.hidden
    cx, sx, dcx, dsx = _quantize(x.reshape(-1, C), qtype)
    ck, sk, dck, dsk = _quantize(np.ascontiguousarray(wk.T), qtype)
    cv, sv, dcv, dsv = _quantize(np.ascontiguousarray(wv.T), qtype)
    log(f"recache_q8 {qtype}")
    swk.sa_cache_recache_q8(gs.cache, dcx, dsx, dck, dsk, dcv, dsv, _qcode(qtype), C)
    torch.cuda.synchronize()
    xd = oquant.dequantize(cx, sx, qtype).reshape(x.shape)
    gs.oracle.recache(xd, oquant.dequantize(ck, sk, qtype).T, oquant.dequantize(cv, sv, qtype).T)
    res = gs.oracle.resident()
    for idx in (0, 3, len(res) - 1):
        ko, vo = _read_frame(gs, idx)
        kref, vref = gs.oracle.frame_kv(res[idx])
        rk, _ = assert_close(to_np(ko), kref, "bf16", f"recached K frame {res[idx]}")
        rv, _ = assert_close(to_np(vo), vref, "bf16", f"recached V frame {res[idx]}")
        log(f"  frame {res[idx]}: K rel_l2 {rk:.2e}, V rel_l2 {rv:.2e}")
    rows = sample_rows(T, T, n=64, seed=5)
    for f in (30, 31):
        q = wl.frame_qkv(w, f, tensor=wl.TENSOR_Q)
        gs.append(wl.frame_qkv(w, f, tensor=wl.TENSOR_K), wl.frame_qkv(w, f, tensor=wl.TENSOR_V), 1, f)
        o = gs.attend(q, 1, swk.SA_MASK_FRAME_CAUSAL)
        _check(gs, q, o, True, rows=rows, what=f"{qtype} recache, frame {f}")


SMALL = wl.Workload("q8-small", 48, batch=2, n_heads=4, head_dim=128, dims=(44, 42, 42), grid=(4, 10),
                    n_sink=2, n_local=3, chunk=1, frames=8, dtype="bf16", sigma=0.8, hidden=256)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("cache,hidden", [("bf16", 256), ("fp8", 256), ("bf16", 192)])
def test_project_append_q8_stream(qtype, cache, hidden):
    """8-bit per-frame projections streamed in chunks of 1-3 frames (sinks, ring wrap, eviction): q, the
    stored K and V and the slot map vs the oracle on the dequantized operands; an e4m3 cache too.  Hidden
    256 is four 64-byte reduction slices, hidden 192 three (a whole number of register-buffer rounds)."""
    import dataclasses
    import torch
    swk = _swk()
    w = dataclasses.replace(SMALL, hidden=hidden)
    eps = wl.head_jitter(w)
    gs = GpuStream(w, eps=eps)
    if cache == "fp8":
        gs.cache = swk.Cache(gs.rope, w.batch, w.n_sink, w.n_local, torch.float8_e4m3fn, k_scale=0.25, v_scale=0.125)
    wq, wk, wv = wl.projection_weights(w)
    C, T = w.hidden, w.tokens_per_frame
    qs = [_quantize(np.ascontiguousarray(m.T), qtype) for m in (wq, wk, wv)]
    deq = [oquant.dequantize(c, s, qtype).T for (c, s, _, _) in qs]
    f0 = 0
    for c in [1, 2, 1, 3, 1]:
        x = wl.frame_hidden(w, f0, c)
        cx, sx, dcx, dsx = _quantize(x.reshape(-1, C), qtype)
        q_out = torch.empty((w.batch, c * T, w.n_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        swk.sa_cache_project_append_q8(gs.cache, dcx, dsx, qs[0][2], qs[0][3], qs[1][2], qs[1][3], qs[2][2],
                                       qs[2][3], _qcode(qtype), C, q_out, c, f0)
        torch.cuda.synchronize()
        xd = oquant.dequantize(cx, sx, qtype).reshape(x.shape)
        q_ref, _ = oproject.project_append(gs.oracle, xd, deq[0], deq[1], deq[2], w.n_heads, f0)
        assert_close(to_np(q_out), q_ref, "bf16", f"{qtype} q of frames {f0}..{f0 + c - 1}")
        assert [(s.frame, s.t, s.segment, s.slot) for s in swk.sa_cache_slots(gs.cache)] == \
            [(s.frame, s.t, s.segment, s.slot) for s in gs.oracle.model.slots()]
        res = gs.oracle.resident()
        for j in range(c):
            idx = len(res) - c + j
            kref, vref = gs.oracle.frame_kv(res[idx])
            if cache == "bf16":
                ko, vo = _read_frame(gs, idx)
                assert_close(to_np(ko), kref, "bf16", f"K of frame {res[idx]}")
                assert_close(to_np(vo), vref, "bf16", f"V of frame {res[idx]}")
            else:
                shape = (w.batch, T, w.n_heads, w.head_dim)
                ko = torch.empty(shape, dtype=torch.uint8, device="cuda")
                vo = torch.empty_like(ko)
                swk.sa_cache_read(gs.cache, idx, ko, vo)
                torch.cuda.synchronize()
                from oracle import fp8 as ofp8
                # the GEMM's own error before the roundings: none for int8 (exact sums); for e4m3 the fp32
                # summation bound C u sum_c |x_c w_c| (u = 2^-24), summed over a RoPE pair for K
                xs = np.abs(xd.reshape(w.batch, c * T, C)[:, j * T:(j + 1) * T])
                slack = {}
                for nm, m in (("K", deq[1]), ("V", deq[2])):
                    sab = (xs @ np.abs(m)).reshape(w.batch, T, w.n_heads, w.head_dim) * C * 2.0 ** -24
                    if qtype == "int8":
                        sab = sab * 0.0
                    if nm == "K":
                        pair = sab[..., 0::2] + sab[..., 1::2]
                        sab = np.repeat(pair, 2, axis=-1)
                    slack[nm] = sab
                for got, ref, sc, nm in ((ko, kref, 0.25, "K"), (vo, vref, 0.125, "V")):
                    val = sc * ofp8.decode(got.cpu().numpy())
                    # e4m3 of a bf16-rounded product: half an e4m3 step plus half a bf16 step
                    err = np.abs(val - ref)
                    bound = (np.abs(ref) + slack[nm]) * (2.0 ** -4 + 2.0 ** -8) * 1.01 + sc * 2.0 ** -10 + slack[nm]
                    assert np.all(err <= bound), f"{nm} of frame {res[idx]}: worst excess {(err - bound).max()}"
        f0 += c


def test_q8_errors():
    """Wrong qtype, an fp32 cache, hidden not a multiple of 64, recache on an empty cache; state unchanged."""
    import torch
    swk = _swk()
    w = SMALL
    gs = GpuStream(w)
    C, T, F = w.hidden, w.tokens_per_frame, w.n_heads * w.head_dim
    xc = torch.zeros((w.batch * T, C), dtype=torch.uint8, device="cuda")
    xs = torch.ones(w.batch * T, dtype=torch.float32, device="cuda")
    wc = torch.zeros((F, C), dtype=torch.uint8, device="cuda")
    ws = torch.ones(F, dtype=torch.float32, device="cuda")
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_recache_q8(gs.cache, xc, xs, wc, ws, wc, ws, swk.SA_Q_INT8, C)
    assert e.value.status == swk.SA_ERR_STATE
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_project_append_q8(gs.cache, xc, xs, None, None, wc, ws, wc, ws, 7, C, None, 1, 0)
    assert e.value.status == swk.SA_ERR_DTYPE
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_project_append_q8(gs.cache, xc, xs, None, None, wc, ws, wc, ws, swk.SA_Q_INT8, 96, None, 1, 0)
    assert e.value.status == swk.SA_ERR_SHAPE
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_project_append_q8(gs.cache, xc, xs, wc, None, wc, ws, wc, ws, swk.SA_Q_INT8, C, None, 1, 0)
    assert e.value.status == swk.SA_ERR_NULL
    assert swk.sa_cache_counts(gs.cache) == (0, 0)
    w32 = wl.Workload("q8-f32", 49, batch=1, n_heads=2, head_dim=64, dims=(22, 22, 20), grid=(8, 8),
                      n_sink=1, n_local=2, chunk=1, frames=2, dtype="f32", hidden=64)
    g32 = GpuStream(w32)
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_cache_project_append_q8(g32.cache, xc, xs, None, None, wc, ws, wc, ws, swk.SA_Q_E4M3, 64, None, 1, 0)
    assert e.value.status == swk.SA_ERR_DTYPE
