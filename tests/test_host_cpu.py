"""CPU tests of the host side: exported C-ABI symbols, host RoPE tables,
argument validation that needs no device, and the cache plan (g++ harness)
against the oracle's cache model."""
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import cache as ocache
from oracle import diagnostics as odiag
from oracle import rope as orope

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")


def _swk():
    import sink_window_kv_amd as swk
    if not os.path.exists(swk.LIB_PATH):
        from sink_window_kv_amd import build
        build.build()
    return swk


def test_library_exports_every_declared_symbol():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", src)))
    assert len(names) >= 18
    lib = _swk().lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"symbols declared but not exported: {missing}"
    assert _swk().sa_version().startswith("libsinkattn")


@pytest.mark.parametrize("sigma,axes,names", [(0.0, 1, ("t",)), (0.8, 1, ("t",)), (0.8, 7, ("t", "h", "w")),
                                              (0.3, 6, ("h", "w"))])
def test_host_rope_tables_match_oracle(sigma, axes, names):
    swk = _swk()
    eps = np.random.default_rng(3).uniform(-1, 1, 12)
    th, fr = swk.sa_rope_tables(12, 128, (44, 42, 42), (30, 52), 10000.0, sigma, eps, axes)
    bases = orope.theta_hat(10000.0, sigma, eps, jitter_axes=names)
    np.testing.assert_allclose(np.array(th), bases, rtol=1e-15)
    for h in range(12):
        np.testing.assert_allclose(fr[h], orope.head_frequencies(bases[h], (44, 42, 42)), rtol=1e-14)


def test_host_rope_theta_table_path():
    """A per-head, per-axis theta_hat table given directly: the eps form's own theta_hat gives the same tables,
    and an arbitrary per-axis table gives the oracle's frequencies (LoL review, method steps (4)-(5))."""
    swk = _swk()
    dims = (44, 42, 42)
    eps = np.random.default_rng(7).uniform(-1, 1, 12)
    for axes, names in ((1, ("t",)), (7, ("t", "h", "w")), (6, ("h", "w"))):
        th_eps, fr_eps = swk.sa_rope_tables(12, 128, dims, (30, 52), 10000.0, 0.8, eps, axes)
        th_tab, fr_tab = swk.sa_rope_tables(12, 128, dims, (30, 52), theta=th_eps)
        assert th_tab == th_eps and fr_tab == fr_eps
    # arbitrary bases, every axis and head different (not expressible as theta0 (1 + sigma eps))
    bases = np.random.default_rng(8).uniform(50.0, 40000.0, size=(12, 3))
    th, fr = swk.sa_rope_tables(12, 128, dims, (30, 52), theta0=2.0, sigma=5.0, eps=None, jitter_axes=0,
                                t_scale=0.5, theta=bases)
    np.testing.assert_array_equal(np.array(th), bases)
    for h in range(12):
        ref = orope.head_frequencies(bases[h], dims)
        ref[:dims[0] // 2] *= 0.5
        np.testing.assert_allclose(fr[h], ref, rtol=1e-14)
    got = np.array(swk.sa_rope_phase_coherence(12, 128, dims, (30, 52), [0, 1, 7, 1200], theta=bases))
    np.testing.assert_allclose(got, odiag.phase_coherence(bases, dims, [0, 1, 7, 1200]), rtol=0, atol=1e-12)
    for bad in (1.0, 0.5, float("nan"), float("inf")):
        b = bases.copy()
        b[5, 2] = bad
        with pytest.raises(swk.SinkAttnError) as e:
            swk.sa_rope_tables(12, 128, dims, (30, 52), theta=b)
        assert e.value.status == swk.SA_ERR_RANGE and "head 5, axis 2" in str(e.value)


def test_host_launch_override_validation():
    """sa_set_launch_override accepts each knob's set (0 = automatic) and rejects the rest."""
    swk = _swk()
    L = swk.lib()
    for knob, good, bad in ((swk.SA_KNOB_ATTN_KERNEL, (0, 1, 2, 3), (4, 8, -1)),
                            (swk.SA_KNOB_ATTN_SPLITS, (0, 1, 3, 16), (-1, 17)),
                            (swk.SA_KNOB_PROJ_TILE, (0, 1, 2, 3, 4), (-1, 5))):
        for v in good:
            assert L.sa_set_launch_override(knob, v) == swk.SA_OK
        for v in bad:
            assert L.sa_set_launch_override(knob, v) == swk.SA_ERR_RANGE
        assert L.sa_set_launch_override(knob, 0) == swk.SA_OK
    assert L.sa_set_launch_override(3, 0) == swk.SA_ERR_RANGE


@pytest.mark.parametrize("sigma,axes,names,dims", [(0.8, 1, ("t",), (44, 42, 42)), (0.0, 1, ("t",), (44, 42, 42)),
                                                   (0.8, 7, ("t", "h", "w"), (22, 22, 20))])
def test_host_phase_coherence_matches_oracle(sigma, axes, names, dims):
    """The library's host C_h(delta) over each head's time frequencies equals the oracle's."""
    swk = _swk()
    D = sum(dims)
    eps = np.random.default_rng(5).uniform(-1, 1, 12)
    deltas = [0, 1, 2, 3, 11, 132, 201, 1200, -7]
    got = np.array(swk.sa_rope_phase_coherence(12, D, dims, (30, 52), deltas, 10000.0, sigma, eps, axes))
    ref = odiag.phase_coherence(orope.theta_hat(10000.0, sigma, eps, jitter_axes=names), dims, deltas)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_rope_phase_coherence(12, 128, (0, 64, 64), (30, 52), deltas)
    assert e.value.status == swk.SA_ERR_SHAPE


@pytest.mark.parametrize("t_scale", [0.25, 0.1, 3.0])
def test_host_position_interpolation_tables_and_coherence(t_scale):
    """t_scale scales the time-axis frequencies only; C(delta) equals the oracle's under PI; 0 means 1."""
    swk = _swk()
    eps = np.random.default_rng(4).uniform(-1, 1, 12)
    dims = (44, 42, 42)
    _, fr = swk.sa_rope_tables(12, 128, dims, (30, 52), 10000.0, 0.8, eps, 1, t_scale)
    bases = orope.theta_hat(10000.0, 0.8, eps)
    for h in range(12):
        ref = orope.head_frequencies(bases[h], dims)
        ref[:dims[0] // 2] *= t_scale
        np.testing.assert_allclose(fr[h], ref, rtol=1e-14)
    assert swk.sa_rope_tables(12, 128, dims, (30, 52), 10000.0, 0.8, eps, 1, 0.0) == \
        swk.sa_rope_tables(12, 128, dims, (30, 52), 10000.0, 0.8, eps, 1)
    deltas = [0, 1, 3, 132, 201, 1200]
    got = np.array(swk.sa_rope_phase_coherence(12, 128, dims, (30, 52), deltas, 10000.0, 0.8, eps, 1, t_scale))
    np.testing.assert_allclose(got, odiag.phase_coherence(bases, dims, deltas, t_scale=t_scale), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kw,status", [
    (dict(t_scale=-0.5), 6), (dict(t_scale=float("inf")), 6), (dict(t_scale=float("nan")), 6),
    (dict(head_dim=96), 2), (dict(dims=(44, 42, 40)), 2), (dict(dims=(43, 43, 42)), 2),
    (dict(grid=(3, 3)), 2), (dict(theta0=1.0), 6), (dict(sigma=-0.1), 6),
    (dict(eps=[1.5] * 12), 6), (dict(sigma=1.0, eps=[-1.0] * 12), 6), (dict(jitter_axes=8), 6),
])
def test_host_rope_validation(kw, status):
    swk = _swk()
    args = dict(n_heads=12, head_dim=128, dims=(44, 42, 42), grid=(30, 52), theta0=10000.0, sigma=0.8,
                eps=[0.0] * 12, jitter_axes=1)
    args.update(kw)
    with pytest.raises(swk.SinkAttnError) as e:
        swk.sa_rope_tables(**args)
    assert e.value.status == status
    assert swk.lib().sa_last_error().decode() != ""


def test_host_cache_store_bytes_and_null_checks():
    import ctypes
    swk = _swk()
    d = swk.sa_cache_desc()
    d.batch, d.n_heads, d.head_dim, d.tokens_per_frame, d.n_sink, d.n_local, d.dtype = 1, 12, 128, 1560, 3, 9, 0
    assert swk.lib().sa_cache_store_bytes(ctypes.byref(d)) == 12 * 12 * 1560 * 128 * 2
    d.dtype = 1
    assert swk.lib().sa_cache_store_bytes(ctypes.byref(d)) == 12 * 12 * 1560 * 128 * 4
    assert swk.lib().sa_cache_bytes(ctypes.byref(d)) == swk.lib().sa_cache_store_bytes(ctypes.byref(d))
    d.n_local = 0
    assert swk.lib().sa_cache_store_bytes(ctypes.byref(d)) == 0
    assert swk.lib().sa_cache_bytes(ctypes.byref(d)) == 0
    d.n_local, d.n_sink = 60, 5
    assert swk.lib().sa_cache_store_bytes(ctypes.byref(d)) == 0
    h = ctypes.c_void_p()
    assert swk.lib().sa_cache_create(None, None, ctypes.byref(h)) == swk.SA_ERR_NULL
    assert swk.lib().sa_window_attn(None, None, None, 1, 0.0, 0, None, 0, None) == swk.SA_ERR_NULL
    assert swk.lib().sa_cache_append(None, None, None, 1, 0, None) == swk.SA_ERR_NULL
    assert swk.lib().sa_status_str(6) == b"SA_ERR_RANGE"


# The host slot plan is built twice: plainly, and (host code only, g++) with
# AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer, any report
# failing the run.
_SANITIZE = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module", params=["plain", "sanitized"])
def plan_harness(request):
    exe = os.path.join(tempfile.mkdtemp(prefix="swk_plan_"), "plan_harness")
    extra = _SANITIZE if request.param == "sanitized" else []
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", *extra,
                    "-I", os.path.join(ROOT, "sink_window_kv_amd", "csrc"),
                    os.path.join(ROOT, "tests", "cpp", "plan_harness.cpp"), "-o", exe], check=True)
    return exe


def _run_plan(exe, n_sink, n_local, cmds):
    inp = f"{n_sink} {n_local}\n" + "\n".join(cmds) + "\n"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    r = subprocess.run([exe], input=inp, capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"plan harness exited {r.returncode}:\n{r.stderr[-2000:]}"
    out = r.stdout
    rows = []
    for line in out.strip().splitlines():
        parts = line.split()
        ents = [tuple(int(x) for x in p.split(",")) for p in parts[2:]]
        rows.append((int(parts[0]), int(parts[1]), ents))
    return rows


@pytest.mark.parametrize("n_sink,n_local,chunk", [(1, 2, 1), (3, 9, 1), (3, 9, 3), (0, 5, 2), (2, 4, 3), (0, 64, 7)])
def test_cache_plan_matches_oracle_model(plan_harness, n_sink, n_local, chunk):
    cmds, t0s = [], []
    t = 0
    for f0 in range(0, 40, chunk):
        cmds.append(f"a {chunk} {t}")
        t0s.append(t)
        t += chunk + (f0 % 3)  # gaps between chunks are allowed; consecutive inside a chunk
    rows = _run_plan(plan_harness, n_sink, n_local, cmds)
    m = ocache.CacheModel(n_sink, n_local)
    for (code, n_app, ents), t0 in zip(rows, t0s):
        m.append(chunk, t0)
        assert code == 0 and n_app == m.n_appended
        assert ents == [(e.frame, e.t, e.segment, e.slot) for e in m.slots()]


def test_cache_plan_rejections_and_reset(plan_harness):
    rows = _run_plan(plan_harness, 3, 9, ["a 3 0", "a 10 3", "a 1 2", "a 0 9", "a 9 3", "r", "a 1 0"])
    assert [r[0] for r in rows] == [0, 2, 3, 1, 0, 0, 0]
    assert rows[4][1] == 12 and rows[5][1] == 0 and rows[6][2] == [(0, 0, 0, 0)]


def test_host_q8_validation():
    """Argument checks of the 8-bit entry points that fail before any launch (no call reaches the GPU)."""
    swk = _swk()
    L = swk.lib()
    P, Q, R, S1, S2 = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    I8, E4 = swk.SA_Q_INT8, swk.SA_Q_E4M3
    assert L.sa_quantize_rows(None, Q, S1, I8, 4, 64, None) == swk.SA_ERR_NULL
    assert L.sa_quantize_rows(P, Q, S1, 5, 4, 64, None) == swk.SA_ERR_DTYPE
    assert L.sa_quantize_rows(P, Q + 4, S1, I8, 4, 64, None) == swk.SA_ERR_ALIGN
    assert L.sa_quantize_rows(P, Q, S1, E4, 4, 60, None) == swk.SA_ERR_SHAPE      # cols % 8
    assert L.sa_quantize_rows(P, Q, S1, E4, -1, 64, None) == swk.SA_ERR_SHAPE
    assert L.sa_quantize_rows(P, Q, S1, I8, 0, 64, None) == swk.SA_OK             # nothing to do
    assert L.sa_quantize_rows(P, P + 4 * 64, S1, I8, 4, 64, None) == swk.SA_ERR_RANGE   # codes inside x
    assert L.sa_quantize_rows(P, Q, P + 16, I8, 4, 64, None) == swk.SA_ERR_RANGE        # scales inside x
    assert L.sa_quantize_rows(P, Q, Q + 128, E4, 4, 64, None) == swk.SA_ERR_RANGE       # scales inside codes
    assert L.sa_quantize_rows(P, P, S1, I8, 4, 64, None) == swk.SA_ERR_RANGE            # in place
    assert L.sa_linear_q8(P, S1, Q, S2, None, I8, 4, 64, 64, None) == swk.SA_ERR_NULL
    assert L.sa_linear_q8(P, S1, Q, S2, R, 9, 4, 64, 64, None) == swk.SA_ERR_DTYPE
    assert L.sa_linear_q8(P, S1 + 4, Q, S2, R, I8, 4, 64, 64, None) == swk.SA_ERR_ALIGN
    assert L.sa_linear_q8(P, S1, Q, S2, R, I8, 4, 96, 64, None) == swk.SA_ERR_SHAPE   # in % 64
    assert L.sa_linear_q8(P, S1, Q, S2, R, E4, 4, 64, 40, None) == swk.SA_ERR_SHAPE   # out % 16
    assert L.sa_linear_q8(P, S1, Q, S2, P + 64, I8, 4, 64, 64, None) == swk.SA_ERR_RANGE  # y overlaps x
    assert L.sa_linear_q8(P, S1, Q, S2, S2, E4, 4, 64, 64, None) == swk.SA_ERR_RANGE      # y overlaps w_scales
    assert L.sa_linear_q8(P, S1, Q, S2, R, E4, 0, 64, 64, None) == swk.SA_OK
    assert L.sa_cache_recache_q8(None, P, S1, Q, S2, R, S2, I8, 64, None) == swk.SA_ERR_NULL
    assert L.sa_cache_project_append_q8(None, P, S1, None, None, Q, S2, R, S2, I8, 64, None, 1, 0, None) == \
        swk.SA_ERR_NULL


def test_host_projection_validation():
    """Argument checks of sa_linear / sa_cache_project_append that fail before any launch."""
    L = _swk().lib()
    P, Q, R = 0x100000, 0x200000, 0x300000   # 16-byte aligned stand-ins; no call below reaches the GPU
    assert L.sa_linear(None, Q, R, 0, 4, 64, 64, None) == _swk().SA_ERR_NULL
    assert L.sa_linear(P, Q, R + 8, 0, 4, 64, 64, None) == _swk().SA_ERR_ALIGN
    assert L.sa_linear(P, Q, R, 7, 4, 64, 64, None) == _swk().SA_ERR_DTYPE
    assert L.sa_linear(P, Q, R, 0, 4, 48, 64, None) == _swk().SA_ERR_SHAPE     # in % 32
    assert L.sa_linear(P, Q, R, 0, 4, 64, 24, None) == _swk().SA_ERR_SHAPE     # out % 16
    assert L.sa_linear(P, Q, R, 0, -1, 64, 64, None) == _swk().SA_ERR_SHAPE
    assert L.sa_linear(P, Q, R, 0, 1 << 26, 64, 64, None) == _swk().SA_ERR_SHAPE   # x reaches 4 GiB
    assert L.sa_linear(P, Q, P + 256, 0, 4, 64, 64, None) == _swk().SA_ERR_RANGE   # y overlaps x
    assert L.sa_linear(P, Q, Q, 0, 4, 64, 64, None) == _swk().SA_ERR_RANGE         # y overlaps w
    assert L.sa_linear(P, Q, R, 0, 0, 64, 64, None) == _swk().SA_OK                # nothing to do
    assert L.sa_cache_project_append(None, P, None, Q, R, 64, None, 1, 0, None) == _swk().SA_ERR_NULL


def test_bench_rejects_more_than_one_gpu():
    """`bench.py --gpus N` with N > 1 exits with status 2 and a JSON error line, before touching a GPU."""
    import json
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
