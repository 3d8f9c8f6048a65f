"""Benchmark: sink + window attention on one MI355X (Wan-1.3B-shaped layer, bf16).

One step = one latent frame of one layer in steady state, the whole hot path:
  sa_cache_append  (K rotated at the frame's time and written to its ring slot,
                    V written transposed; the oldest local frame is evicted)
  sa_window_attn   (the frame's 1560 queries, rotated on load, attend over
                    3 sink + 9 local frames = 18720 keys, 12 heads, D = 128).
Steps cycle over 8 independent layer caches (8 x 115 MB, larger than the
256 MB last-level cache) so K/V come from HBM as in a real layer stack.

The KV recache (prompt switch, M = 18720 tokens, N = 2 x 1536, K = 1536) and
the standalone RoPE are timed in the same run and reported beside the step.

value = attention algorithmic TFLOP/s of the whole step (4 H D per visible
query-key pair = 179.42 GFLOP per frame; the append's time counts, its bytes
add no flops).  roofline.achieved uses the attention kernel's own time from
HIP events around each call on the launch stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (vendor figure)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 (e4m3) MFMA (vendor figure)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
N_LAYERS = 8


def attn_flops(n_q_rows: int, n_keys: int, H: int, D: int) -> float:
    return 4.0 * H * D * n_q_rows * n_keys


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the shader-clock sample (rocm-smi, a child process): for runs under a counter "
                         "profiler, whose preloaded library has initialised the GPU in every child")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy three times (HBM counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    """A copy kernel of known size: reads and writes 512 MiB per launch.  Its
    FETCH_SIZE / WRITE_SIZE counters give the scale from counter KiB to HBM bytes."""
    import torch
    n = 128 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": 4 * n, "copy_bytes_written_per_launch": 4 * n}), flush=True)


ATTN_BF16_SOURCES = [os.path.join(ROOT, "sink_window_kv_amd", "csrc", f)
                     for f in ("window_attn.hip", "attn_common.hpp", "device_common.hpp", "internal.hpp")]


def code_digest(src_paths) -> str:
    """sha256[:16] of C++/HIP sources (concatenated) with comments and blank lines
    removed, so that editing a comment does not orphan counters taken on the same code."""
    import re
    if isinstance(src_paths, str):
        src_paths = [src_paths]
    text = "\n".join(open(p).read() for p in src_paths)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profile(kernel_srcs):
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current kernel code (else None)."""
    path = os.path.join(ROOT, "profiles", "attn_bf16_wan13b_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if (vals.get("kernel_code_sha256_16") or "").split(" ")[0] != code_digest(kernel_srcs):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_of_step(kernel_srcs):
    """Kernel-only durations of the bench step's attention call from the committed kernel-trace summary,
    with the shader clock and box it was taken on, if it was taken on the current kernel code (else None)."""
    path = os.path.join(ROOT, "profiles", "attn_bf16_wan13b_kernel_trace.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = v.strip().split("  ")[0].strip()
    if vals.get("kernel_code_sha256_16") != code_digest(kernel_srcs):
        return None
    try:
        att, mrg = float(vals["step_attention_kernel_mean_us"]), float(vals["step_merge_kernel_mean_us"])
        sclk = int(vals["sclk_mhz_under_load"]) if vals.get("sclk_mhz_under_load", "").isdigit() else None
    except (KeyError, ValueError):
        return None
    return {"attention_kernel_us": att, "merge_kernel_us": mrg, "call_us": round(att + mrg, 2),
            "sclk_mhz": sclk, "box": vals.get("box")}


def sclk_under_load(launch, n_calls: int):
    """Shader clock (MHz) that rocm-smi reports while n_calls launches run, or None."""
    import re
    import subprocess
    import threading
    import torch
    got = {}

    def sample():
        time.sleep(0.3)
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
            m = re.search(r"sclk clock speed:\"?\s*:\s*\"\((\d+)Mhz\)", r.stdout)
            got["mhz"] = int(m.group(1)) if m else None
        except Exception:
            got["mhz"] = None
    torch.cuda.synchronize()
    th = threading.Thread(target=sample)
    for i in range(n_calls // 10):
        launch(i)
    th.start()
    for i in range(n_calls // 10, n_calls):
        launch(i)
    th.join()
    torch.cuda.synchronize()
    return got.get("mhz")


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle as it stands, on a bounded sample of one steady-state step."""
    import numpy as np
    import workloads as wl
    from oracle import attention as oattn
    from oracle import cache as ocache
    from oracle import rope as orope
    cores = _cores()
    T = w.tokens_per_frame
    bases = orope.theta_hat(w.theta0, w.sigma, np.zeros(w.n_heads))
    f0 = 20
    # Steady-state frames f0, f0+1, ...: each rotates its new frame's keys
    # (append) and its queries, then attends head by head, until the budget
    # is spent (checked after every head).  Only oracle calls are on the
    # clock; drawing the seeded inputs is not.
    k_rot, v_raw = {}, {}
    heads_done, f, dt = 0, f0, 0.0
    while dt <= budget_s:
        res = ocache.resident_frames(f + 1, w.n_sink, w.n_local)
        new_k = {r: wl.frame_qkv(w, r, tensor=wl.TENSOR_K) for r in res if r not in k_rot}
        for r in new_k:
            v_raw[r] = wl.frame_qkv(w, r, tensor=wl.TENSOR_V)
        q = wl.frame_qkv(w, f, tensor=wl.TENSOR_Q)
        t0 = time.perf_counter()
        for r, k in new_k.items():
            k_rot[r] = orope.rope3d_frame(k, r, bases, w.dims, w.grid[1])
        q_rot = orope.rope3d_frame(q, f, bases, w.dims, w.grid[1])
        dt += time.perf_counter() - t0
        for h in range(w.n_heads):
            t0 = time.perf_counter()
            oattn.window_attention(q_rot, [k_rot[r] for r in res], [v_raw[r] for r in res], res, [f], T, True,
                                   heads=[h])
            dt += time.perf_counter() - t0
            heads_done += 1
            if dt > budget_s:
                break
        for r in [r for r in k_rot if r not in res]:
            del k_rot[r], v_raw[r]
        f += 1
    n_keys = (w.n_sink + w.n_local) * T
    flops = attn_flops(T, n_keys, heads_done, w.head_dim)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads_done} head-frames ({heads_done / w.n_heads:.2f} steady-state frames from frame {f0}, "
                      f"1560 queries x {n_keys} keys each), fp64 numpy incl. the RoPE of every key and query frame "
                      f"it used; {dt:.1f} s of oracle time (input drawing excluded)",
            "latent_frames_per_s_per_layer": (heads_done / w.n_heads) / dt}


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_recache_leg(w4):
    """The fp64 oracle's KV recache of one Wan-1.3B layer cache (x [18720 x 1536] . W_k, W_v, RoPE of the
    12 frames' keys), the prompt-switch workload; one whole recache, timed once (input drawing excluded)."""
    import numpy as np
    import workloads as wl
    from oracle import recache as orecache
    from oracle import rope as orope
    x, wk, wv = wl.recache_inputs(w4)
    n = w4.n_sink + w4.n_local
    bases = orope.theta_hat(w4.theta0, w4.sigma, np.zeros(w4.n_heads))
    t0 = time.perf_counter()
    orecache.recache(x, wk, wv, w4.n_heads, list(range(18, 18 + n)), w4.tokens_per_frame, bases, w4.dims,
                     w4.grid[1])
    dt = time.perf_counter() - t0
    flops = 2.0 * x.shape[1] * (2 * w4.n_heads * w4.head_dim) * w4.hidden
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "seconds_per_recache": round(dt, 3),
            "sample": f"one whole recache: x [{x.shape[1]} x {w4.hidden}] . W_k, W_v [{w4.hidden} x "
                      f"{w4.n_heads * w4.head_dim}] and the RoPE of the {n} frames' keys, fp64 numpy; timed once"}


def cpu_chunk_leg(w5, budget_s: float):
    """The fp64 oracle on one (stream, layer, 3-frame chunk) of the B = 4 chunked workload in steady state
    (chunk frames 27-29 over sinks 0-2 and local frames 21-29, frame-causal), head by head until the
    budget; extrapolated to the 4-stream layer chunk and to the 30-layer step (x 4 streams x 30 layers)."""
    import numpy as np
    import workloads as wl
    from oracle import attention as oattn
    from oracle import cache as ocache
    from oracle import rope as orope
    T, H, D = w5.tokens_per_frame, w5.n_heads, w5.head_dim
    c, f_last = w5.chunk, 29
    res = ocache.resident_frames(f_last + 1, w5.n_sink, w5.n_local)
    qframes = list(range(f_last - c + 1, f_last + 1))
    bases = orope.theta_hat(w5.theta0, w5.sigma, wl.head_jitter(w5, layer=0))
    one = lambda f, t: wl.normal((1, T, H, D), w5.cfg, 0, 0, f, t, w5.input_scale, w5.dtype)
    k = {f: one(f, wl.TENSOR_K) for f in res}
    v = {f: one(f, wl.TENSOR_V) for f in res}
    q = np.concatenate([one(f, wl.TENSOR_Q) for f in qframes], axis=1)
    t0 = time.perf_counter()
    k_rot = [orope.rope3d_frame(k[f], f, bases, w5.dims, w5.grid[1]) for f in res]
    q_rot = orope.rope3d(q, 0, T, bases, w5.dims, w5.grid[1], t_list=qframes)
    dt = time.perf_counter() - t0
    heads = 0
    while heads < H and dt <= budget_s:
        t0 = time.perf_counter()
        oattn.window_attention(q_rot, k_rot, [v[f] for f in res], res, qframes, T, True, heads=[heads])
        dt += time.perf_counter() - t0
        heads += 1
    per_head = sum(attn_flops(T, (len(res) - c + 1 + i) * T, 1, D) for i in range(c))
    flops = per_head * heads
    stream_chunk_s = dt * H / heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "stream_layer_chunk_s": round(stream_chunk_s, 2),
            "extrapolated_30_layer_step_s": round(stream_chunk_s * w5.batch * 30, 1),
            "latent_frames_per_s_per_layer": w5.batch * c / (stream_chunk_s * w5.batch),
            "sample": f"{heads} of {H} heads of one stream's 3-frame chunk (4680 queries over 10/11/12 frames, "
                      f"frame-causal, sigma 0.8), fp64 numpy incl. the RoPE of the chunk's queries and the resident "
                      f"keys; {dt:.1f} s; the stream-layer-chunk time is extrapolated x {H}/{heads} heads, the "
                      f"30-layer step x 4 streams x 30 layers (extrapolated, not run)"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the kernels shard by head; no multi-GPU path is built); --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import sink_window_kv_amd as swk
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[2]
    T, H, D = w.tokens_per_frame, w.n_heads, w.head_dim
    n_win = w.n_sink + w.n_local
    bf = torch.bfloat16
    print(f"[bench] {w.name}: preparing {N_LAYERS} layer caches", file=sys.stderr, flush=True)

    pool = 16  # distinct seeded frames, reused round-robin
    qs, ks, vs = [], [], []
    for f in range(pool):
        qs.append(torch.from_numpy(wl.frame_qkv(w, f, tensor=wl.TENSOR_Q)).to(dev, bf).contiguous())
        ks.append(torch.from_numpy(wl.frame_qkv(w, f, tensor=wl.TENSOR_K)).to(dev, bf).contiguous())
        vs.append(torch.from_numpy(wl.frame_qkv(w, f, tensor=wl.TENSOR_V)).to(dev, bf).contiguous())
    rope = swk.Rope(H, D, w.dims, w.grid, w.theta0, w.sigma, None)
    caches = [swk.Cache(rope, 1, w.n_sink, w.n_local, bf, device=dev) for _ in range(N_LAYERS)]
    t_next = [0] * N_LAYERS
    for li, c in enumerate(caches):
        for f in range(n_win):
            swk.sa_cache_append(c, ks[(f + li) % pool], vs[(f + li) % pool], 1, t_next[li])
            t_next[li] += 1
    ws_bytes = max(swk.sa_window_attn_workspace(c, 1) for c in caches)
    ws = torch.zeros(max(ws_bytes // 4, 4), dtype=torch.float32, device=dev)
    o = torch.empty_like(qs[0])
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        li = i % N_LAYERS
        c = caches[li]
        fi = (t_next[li] + li) % pool
        if ev is not None:
            ev[0].record(stream)
        swk.sa_cache_append(c, ks[fi], vs[fi], 1, t_next[li])
        if ev is not None:
            ev[1].record(stream)
        swk.sa_window_attn(c, qs[fi], o, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws)
        if ev is not None:
            ev[2].record(stream)
        t_next[li] += 1

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    # Timed region: whole steps, no events in the way.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Same loop again with HIP events on the launch stream: per-kernel durations.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    app_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    att_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    app_avg = sum(app_ms) / len(app_ms)
    att_avg = sum(att_ms) / len(att_ms)

    # Shader clock under this load: about a second of attention calls queued,
    # rocm-smi read once while they run (null if the tool is not there).
    sclk_mhz = None if args.no_sclk else sclk_under_load(
        lambda i: swk.sa_window_attn(caches[i % N_LAYERS], qs[i % pool], o, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws),
        n_calls=6000)

    flops = attn_flops(T, n_win * T, H, D)
    ms_per_step = elapsed * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (att_avg * 1e-3) / 1e12
    append_bytes = 2 * 2 * T * H * D * 2  # K and V, read + write, bf16
    print(f"[bench] step {ms_per_step * 1e3:.1f} us, attention {att_avg * 1e3:.1f} us "
          f"({achieved:.0f} TFLOP/s), append {app_avg * 1e3:.1f} us; shader clock under load {sclk_mhz} MHz",
          file=sys.stderr, flush=True)

    # LoL diagnostic: the same attention call also reporting each row's
    # softmax mass on the sink frames (a second pass over the sink keys).
    # Cycled over the 8 layer caches (0.92 GB) like the step, so K/V come from HBM.
    mass = torch.empty((1, T, H), dtype=torch.float32, device=dev)
    for i in range(3):
        swk.sa_window_attn_sink_mass(caches[i], qs[i], o, mass, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws)
    em0, em1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    em0.record(stream)
    for i in range(24):
        swk.sa_window_attn_sink_mass(caches[i % N_LAYERS], qs[i % pool], o, mass, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws)
    em1.record(stream)
    torch.cuda.synchronize()
    mass_us = em0.elapsed_time(em1) * 1e3 / 24

    # Window-size variants (3, 12 and 24 local frames without sinks; 9 local
    # + 3 sink is the main workload): steady-state attention of one frame.
    # Each variant cycles enough caches (at least 3) for a working set above 300 MB, so K/V come from HBM.
    windows = {}
    for n_s, n_l in ((0, 3), (0, 12), (0, 24)):
        per_cache = 2 * (n_s + n_l) * T * H * D * 2
        n_c = max(3, -(-300_000_000 // per_cache))
        cws = [swk.Cache(rope, 1, n_s, n_l, bf, device=dev) for _ in range(n_c)]
        for ci, cw in enumerate(cws):
            for f in range(n_s + n_l):
                swk.sa_cache_append(cw, ks[(f + ci) % pool], vs[(f + ci) % pool], 1, f)
        wsw = torch.zeros(max(swk.sa_window_attn_workspace(cws[0], 1) // 4, 4), dtype=torch.float32, device=dev)
        for i in range(n_c):
            swk.sa_window_attn(cws[i], qs[i % pool], o, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, wsw)
        n_w = 8 * n_c if n_c < 8 else 2 * n_c
        ew0, ew1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ew0.record(stream)
        for i in range(n_w):
            swk.sa_window_attn(cws[i % n_c], qs[i % pool], o, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, wsw)
        ew1.record(stream)
        torch.cuda.synchronize()
        us_w = ew0.elapsed_time(ew1) * 1e3 / n_w
        fl_w = attn_flops(T, (n_s + n_l) * T, H, D)
        windows[f"{n_s}+{n_l}"] = {"attention_avg_us": round(us_w, 1), "TFLOPs": round(fl_w / (us_w * 1e-6) / 1e12, 1),
                                   "caches_cycled": n_c, "working_set_MB": round(n_c * per_cache / 1e6)}
        for cw in cws:
            cw.close()
    windows["3+9"] = {"attention_avg_us": round(att_avg * 1e3, 1), "TFLOPs": round(achieved, 1)}

    # Standalone RoPE (Q of one frame, read + write) and the KV recache.
    qrot = torch.empty_like(qs[0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(5):
        swk.sa_rope3d_apply(rope, qs[0], qrot, 1, 1, 123)
    e0.record(stream)
    for _ in range(50):
        swk.sa_rope3d_apply(rope, qs[0], qrot, 1, 1, 123)
    e1.record(stream)
    torch.cuda.synchronize()
    rope_us = e0.elapsed_time(e1) * 1e3 / 50
    rope_bytes = 2 * T * H * D * 2

    # The recache cycles 3 hidden-state inputs (3 x 57.5 MB) and 3 layer caches (3 x 115 MB), so its
    # operands come from HBM rather than the 256 MB last-level cache.
    w4 = wl.WORKLOADS[4]
    txs = []
    for bi in range(3):
        x, wk, wv = wl.recache_inputs(w4, base=bi)
        txs.append(torch.from_numpy(x).to(dev, bf).contiguous())
    x, wk, wv = wl.recache_inputs(w4)
    tx = txs[0]
    twk = torch.from_numpy(np.ascontiguousarray(wk.T)).to(dev, bf).contiguous()
    twv = torch.from_numpy(np.ascontiguousarray(wv.T)).to(dev, bf).contiguous()
    rc = caches[0]
    for i in range(3):
        swk.sa_cache_recache(caches[i], txs[i], twk, twv, w4.hidden)
    e0.record(stream)
    n_rc = 21
    for i in range(n_rc):
        swk.sa_cache_recache(caches[i % 3], txs[i % 3], twk, twv, w4.hidden)
    e1.record(stream)
    torch.cuda.synchronize()
    rc_us = e0.elapsed_time(e1) * 1e3 / n_rc
    rc_flops = 2.0 * (n_win * T) * (2 * H * D) * w4.hidden
    rc_bytes = (n_win * T * w4.hidden + 2 * H * D * w4.hidden + 2 * n_win * T * H * D) * 2

    # One layer's self-attention block per frame, hidden 1536: fused Q/K/V
    # projections with RoPE and the append, the attention, and the output
    # projection (seeded random weights of that shape; no model).
    C = w4.hidden
    HD = H * D
    wq_, wk_, wv_ = wl.projection_weights(w4)
    dqw, dkw, dvw = (torch.from_numpy(np.ascontiguousarray(m.T)).to(dev, bf).contiguous() for m in (wq_, wk_, wv_))
    dow = torch.from_numpy(np.ascontiguousarray(wl.output_weight(w4).T)).to(dev, bf).contiguous()
    xs = [torch.from_numpy(wl.frame_hidden(w4, f, 1)).to(dev, bf).contiguous() for f in range(4)]
    cb = swk.Cache(rope, 1, w.n_sink, w.n_local, bf, device=dev)
    qb = torch.empty((1, T, H, D), dtype=bf, device=dev)
    ob = torch.empty_like(qb)
    yb = torch.empty((T, C), dtype=bf, device=dev)
    tb = 0
    for f in range(n_win):
        swk.sa_cache_project_append(cb, xs[f % 4], dqw, dkw, dvw, C, qb, 1, tb)
        tb += 1
    # back to back, one synchronisation at the end (events between the launches)
    n_blk, n_skip = 43, 3
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_blk)]
    for it in range(n_blk):
        ea, eb, ec, ed = bev[it]
        ea.record(stream)
        swk.sa_cache_project_append(cb, xs[it % 4], dqw, dkw, dvw, C, qb, 1, tb)
        eb.record(stream)
        swk.sa_window_attn(cb, qb, ob, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws)
        ec.record(stream)
        swk.sa_linear(ob, dow, yb, T, HD, C)
        ed.record(stream)
        tb += 1
    torch.cuda.synchronize()
    pj_ms = [e[0].elapsed_time(e[1]) for e in bev[n_skip:]]
    ab_ms = [e[1].elapsed_time(e[2]) for e in bev[n_skip:]]
    op_ms = [e[2].elapsed_time(e[3]) for e in bev[n_skip:]]
    pj_avg, ab_avg, op_avg = (sum(v) / len(v) for v in (pj_ms, ab_ms, op_ms))
    pj_flops = 2.0 * T * C * 3 * HD
    op_flops = 2.0 * T * HD * C
    print(f"[bench] layer block: q/k/v projection + append {pj_avg * 1e3:.1f} us "
          f"({pj_flops / (pj_avg * 1e-3) / 1e12:.0f} TFLOP/s), attention {ab_avg * 1e3:.1f} us, "
          f"output projection {op_avg * 1e3:.1f} us ({op_flops / (op_avg * 1e-3) / 1e12:.0f} TFLOP/s)",
          file=sys.stderr, flush=True)
    cb.close()

    # Chunked, batched shape: B = 4 streams, 3-frame query chunks, frame-causal
    # (4680 queries per stream over 10/11/12 visible frames), sigma = 0.8.
    w5 = wl.WORKLOADS[5]
    eps5 = wl.head_jitter(w5, layer=0)
    rope5 = swk.Rope(H, D, w5.dims, w5.grid, w5.theta0, w5.sigma, eps5)
    c5 = swk.Cache(rope5, w5.batch, w5.n_sink, w5.n_local, bf, device=dev)
    chunks5 = []
    for ci in range(4):
        f0 = ci * w5.chunk
        chunks5.append(tuple(torch.from_numpy(wl.chunk_qkv(w5, f0, w5.chunk, 0, t)).to(dev, bf).contiguous()
                             for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V)))
    t5 = 0
    for ci in range(4):  # fill: 12 frames resident after four chunks
        swk.sa_cache_append(c5, chunks5[ci][1], chunks5[ci][2], w5.chunk, t5)
        t5 += w5.chunk
    ws5_bytes = swk.sa_window_attn_workspace(c5, w5.chunk)
    ws5 = torch.zeros(max(ws5_bytes // 4, 4), dtype=torch.float32, device=dev)
    o5 = torch.empty_like(chunks5[0][0])
    a5_ms, ap5_ms = [], []
    for it in range(13):
        q5, k5, v5 = chunks5[it % 4]
        ea, eb, ec = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        ea.record(stream)
        swk.sa_cache_append(c5, k5, v5, w5.chunk, t5)
        eb.record(stream)
        swk.sa_window_attn(c5, q5, o5, w5.chunk, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws5)
        ec.record(stream)
        t5 += w5.chunk
        torch.cuda.synchronize()
        if it >= 3:
            ap5_ms.append(ea.elapsed_time(eb))
            a5_ms.append(eb.elapsed_time(ec))
    # visible keys per query frame i of the chunk: 3 sinks + (7 + i) local frames
    flops5 = sum(attn_flops(T, (w5.n_sink + w5.n_local - (w5.chunk - 1) + i) * T, H, D)
                 for i in range(w5.chunk)) * w5.batch
    a5_avg = sum(a5_ms) / len(a5_ms)
    ap5_avg = sum(ap5_ms) / len(ap5_ms)
    print(f"[bench] B=4 3-frame chunks: attention {a5_avg * 1e3:.1f} us "
          f"({flops5 / (a5_avg * 1e-3) / 1e12:.0f} TFLOP/s), append {ap5_avg * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    c5.close()

    # FP8 (e4m3) cache: the same frame step (append + attention, 8 layer
    # caches cycled) and the B = 4 chunk, with the cache in e4m3.
    f8 = torch.float8_e4m3fn
    c8s = [swk.Cache(rope, 1, w.n_sink, w.n_local, f8, device=dev, k_scale=1.0 / 256, v_scale=1.0 / 256)
           for _ in range(N_LAYERS)]
    t8 = [0] * N_LAYERS
    for li, c in enumerate(c8s):
        for f in range(n_win):
            swk.sa_cache_append(c, ks[(f + li) % pool], vs[(f + li) % pool], 1, t8[li])
            t8[li] += 1
    ws8 = torch.zeros(max(max(swk.sa_window_attn_workspace(c, 1) for c in c8s) // 4, 4), dtype=torch.float32,
                      device=dev)
    n8, skip8 = 120, 20
    ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n8)]
    for i in range(n8):
        li = i % N_LAYERS
        fi = (t8[li] + li) % pool
        ev8[i][0].record(stream)
        swk.sa_cache_append(c8s[li], ks[fi], vs[fi], 1, t8[li])
        ev8[i][1].record(stream)
        swk.sa_window_attn(c8s[li], qs[fi], o, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws8)
        ev8[i][2].record(stream)
        t8[li] += 1
    torch.cuda.synchronize()
    a8 = sum(e[1].elapsed_time(e[2]) for e in ev8[skip8:]) / (n8 - skip8)
    p8 = sum(e[0].elapsed_time(e[1]) for e in ev8[skip8:]) / (n8 - skip8)
    for c in c8s:
        c.close()
    c58 = swk.Cache(rope5, w5.batch, w5.n_sink, w5.n_local, f8, device=dev, k_scale=1.0 / 256, v_scale=1.0 / 256)
    t58 = 0
    for ci in range(4):
        swk.sa_cache_append(c58, chunks5[ci][1], chunks5[ci][2], w5.chunk, t58)
        t58 += w5.chunk
    ws58 = torch.zeros(max(swk.sa_window_attn_workspace(c58, w5.chunk) // 4, 4), dtype=torch.float32, device=dev)
    a58_ms = []
    for it in range(13):
        q5, k5, v5 = chunks5[it % 4]
        swk.sa_cache_append(c58, k5, v5, w5.chunk, t58)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record(stream)
        swk.sa_window_attn(c58, q5, o5, w5.chunk, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws58)
        eb.record(stream)
        t58 += w5.chunk
        torch.cuda.synchronize()
        if it >= 3:
            a58_ms.append(ea.elapsed_time(eb))
    a58 = sum(a58_ms) / len(a58_ms)
    c58.close()
    rope5.close()
    print(f"[bench] fp8 cache: attention {a8 * 1e3:.1f} us ({flops / (a8 * 1e-3) / 1e12:.0f} TFLOP/s), "
          f"append {p8 * 1e3:.1f} us; B=4 chunks {a58 * 1e3:.1f} us ({flops5 / (a58 * 1e-3) / 1e12:.0f} TFLOP/s)",
          file=sys.stderr, flush=True)

    # 8-bit projections (W8A8: int8 or e4m3 codes, fp32 scales per token and
    # per output feature): row quantisation of one frame's hidden states, the
    # output projection, the fused q/k/v projections + append, and the recache.
    q8 = {"workload": "W8A8 projections: codes with one fp32 scale per token (x) and per output feature (W); "
                      "frame shapes of the layer block and the recache (x [18720 x 1536] -> K, V)"}
    qx_bytes = T * C * 3 + T * 4
    def q8_codes(t2d, qt):
        cc = torch.empty(t2d.shape, dtype=torch.uint8, device=dev)
        sc = torch.empty(t2d.shape[0], dtype=torch.float32, device=dev)
        swk.sa_quantize_rows(t2d, cc, sc, qt)
        return cc, sc
    def timed(fn, n, warm=3):
        for _ in range(warm):
            fn()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n
    for qname, qt in (("int8", swk.SA_Q_INT8), ("e4m3", swk.SA_Q_E4M3)):
        x0 = xs[0].reshape(T, C)
        cx0 = torch.empty((T, C), dtype=torch.uint8, device=dev)
        sx0 = torch.empty(T, dtype=torch.float32, device=dev)
        quant_us = timed(lambda: swk.sa_quantize_rows(x0, cx0, sx0, qt), 50)
        cq, sq = q8_codes(dqw, qt)
        ck_, sk_ = q8_codes(dkw, qt)
        cv_, sv_ = q8_codes(dvw, qt)
        co_, so_ = q8_codes(dow, qt)
        out_us = timed(lambda: swk.sa_linear_q8(cx0, sx0, co_, so_, yb, qt, T, C, C), 50)
        cq8 = swk.Cache(rope, 1, w.n_sink, w.n_local, bf, device=dev)
        tq8 = [0]
        def pa():
            swk.sa_cache_project_append_q8(cq8, cx0, sx0, cq, sq, ck_, sk_, cv_, sv_, qt, C, qb, 1, tq8[0])
            tq8[0] += 1
        pa_us = timed(pa, 40, warm=n_win)
        cq8.close()
        cxr, sxr = q8_codes(tx.reshape(-1, C), qt)
        rc_q8_us = timed(lambda: swk.sa_cache_recache_q8(rc, cxr, sxr, ck_, sk_, cv_, sv_, qt, C), 10)
        q8[qname] = {"quantize_frame_us": round(quant_us, 2),
                     "quantize_GBps": round(qx_bytes / (quant_us * 1e-6) / 1e9, 1),
                     "out_proj_us": round(out_us, 1), "out_proj_TOPs": round(op_flops / (out_us * 1e-6) / 1e12, 1),
                     "qkv_append_us": round(pa_us, 1), "qkv_TOPs": round(pj_flops / (pa_us * 1e-6) / 1e12, 1),
                     "recache_us": round(rc_q8_us, 1), "recache_TOPs": round(rc_flops / (rc_q8_us * 1e-6) / 1e12, 1),
                     "recache_pct_8bit_peak": round(100.0 * rc_flops / (rc_q8_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 2)}
        print(f"[bench] {qname} projections: quantize {quant_us:.1f} us, output projection {out_us:.1f} us, "
              f"q/k/v + append {pa_us:.1f} us, recache {rc_q8_us:.1f} us "
              f"({rc_flops / (rc_q8_us * 1e-6) / 1e12:.0f} TOP/s)", file=sys.stderr, flush=True)

    traffic = traffic_from_profile(ATTN_BF16_SOURCES)
    prof = profile_of_step(ATTN_BF16_SOURCES)
    if prof is not None:
        prof["frac_call"] = round(flops / (prof["call_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
        prof["frac_attention_kernel"] = round(flops / (prof["attention_kernel_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if prof["sclk_mhz"] and sclk_mhz:
            # the same call scaled from the profiled box's clock to this run's
            prof["call_us_at_this_clock"] = round(prof["call_us"] * prof["sclk_mhz"] / sclk_mhz, 2)
    out = {
        "metric": "sink+window attn TFLOP/s & latent frames/s/layer on 1 MI355X; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(128) Q, K, V in bf16; no model weights)",
        "config": {"workload": "wan13b-layer-bf16: B=1, H=12, D=128 (RoPE 44/42/42), 30x52=1560 tokens/frame, "
                               "3 sink + 9 local = 18720 keys, 1 query frame, sigma=0; step = append + attend, "
                               "8 layer caches cycled",
                   "layers_cycled": N_LAYERS, "tokens_per_frame": T, "keys": n_win * T},
        "latent_frames_per_s_per_layer": round(1e3 / ms_per_step, 1),
        "attention_only_latent_frames_per_s_per_layer": round(1e3 / att_avg, 1),
        "pct_bf16_peak_step": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "pct_bf16_peak_attention_kernel": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
        "sclk_mhz_under_load": sclk_mhz,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "frac_at_measured_clock": (round(achieved / (PEAK_BF16_TFLOPS * sclk_mhz / 2400.0), 4)
                                                if sclk_mhz else None),
                     "traffic": traffic, "kernel": "attn_bf16_kernel<128>",
                     "flops_per_launch": flops, "avg_launch_us": round(att_avg * 1e3, 2),
                     "median_launch_us": round(att_ms[len(att_ms) // 2] * 1e3, 2),
                     "launch_note": "avg_launch_us: HIP events on the launch stream around each sa_window_attn "
                                    "call of the step (attention kernel + split merge)",
                     "profile": prof},
        "append": {"avg_us": round(app_avg * 1e3, 2), "bytes": append_bytes,
                   "GBps": round(append_bytes / (app_avg * 1e-3) / 1e9, 1), "peak_GBps": PEAK_HBM_GBPS},
        "window_variants": {"note": "sink+local frames; one 1560-query frame, frame-causal, steady state",
                            **windows},
        "sink_mass": {"avg_us": round(mass_us, 1),
                      "vs_attention_only": round(mass_us / (att_avg * 1e3), 3),
                      "note": "sa_window_attn_sink_mass: the attention plus each row's softmax mass on the "
                              "3 sink frames, per head; cycled over the 8 layer caches"},
        "rope3d_q": {"avg_us": round(rope_us, 2), "bytes": rope_bytes,
                     "GBps": round(rope_bytes / (rope_us * 1e-6) / 1e9, 1)},
        "recache": {"avg_us": round(rc_us, 1), "flops": rc_flops,
                    "TFLOPs": round(rc_flops / (rc_us * 1e-6) / 1e12, 1),
                    "pct_bf16_peak": round(100.0 * rc_flops / (rc_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
                    "min_bytes": rc_bytes, "note": "3 hidden-state inputs and 3 layer caches cycled"},
        "layer_block": {"workload": "wan13b self-attention block per frame: x [1560 x 1536] -> fused q/k/v "
                                     "projections + RoPE + append, attention over 12 frames, output projection "
                                     "[1560 x 1536] . [1536 x 1536]",
                        "qkv_append_avg_us": round(pj_avg * 1e3, 1), "qkv_flops": pj_flops,
                        "qkv_TFLOPs": round(pj_flops / (pj_avg * 1e-3) / 1e12, 1),
                        "attention_avg_us": round(ab_avg * 1e3, 1),
                        "out_proj_avg_us": round(op_avg * 1e3, 1), "out_proj_flops": op_flops,
                        "out_proj_TFLOPs": round(op_flops / (op_avg * 1e-3) / 1e12, 1),
                        "latent_frames_per_s_per_layer": round(1e3 / (pj_avg + ab_avg + op_avg), 1)},
        "chunked_b4": {"workload": "wan13b-chunk3-b4: B=4, 3-frame query chunks (4680 queries per stream), "
                                    "frame-causal over 10/11/12 visible frames, sigma=0.8, one layer",
                       "attention_avg_us": round(a5_avg * 1e3, 1), "flops": flops5,
                       "TFLOPs": round(flops5 / (a5_avg * 1e-3) / 1e12, 1),
                       "pct_bf16_peak": round(100.0 * flops5 / (a5_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                       "append_avg_us": round(ap5_avg * 1e3, 1),
                       "latent_frames_per_s_per_layer": round(w5.batch * w5.chunk / ((a5_avg + ap5_avg) * 1e-3), 1)},
        "fp8_cache": {"workload": "the same two workloads with the KV cache in OCP e4m3 (per-tensor scales); "
                                  "q and p rounded to e4m3 in the kernel; bf16 in and out",
                      "attention_avg_us": round(a8 * 1e3, 1),
                      "TFLOPs": round(flops / (a8 * 1e-3) / 1e12, 1),
                      "pct_fp8_peak": round(100.0 * flops / (a8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                      "append_avg_us": round(p8 * 1e3, 1),
                      "latent_frames_per_s_per_layer": round(1e3 / (a8 + p8), 1),
                      "b4_chunk_attention_avg_us": round(a58 * 1e3, 1),
                      "b4_chunk_TFLOPs": round(flops5 / (a58 * 1e-3) / 1e12, 1)},
        "q8_projections": q8,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        out["cpu_baseline"]["recache"] = cpu_recache_leg(w4)
        out["cpu_baseline"]["chunked_b4"] = cpu_chunk_leg(w5, args.cpu_seconds / 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
