"""GPU: SA_DEBUG_SYNC=1 (read when the library loads, so in a child process) makes every entry point wait for
its stream after launching; results must not change.  The child runs an append + attention + recache
stream on a small bf16 cache and saves the outputs; the parent runs the same calls without the variable and
compares bit for bit."""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import sink_window_kv_amd as swk
import workloads as wl
import dataclasses
w = dataclasses.replace(wl.WORKLOADS[2], name="debug-sync", cfg=57, n_heads=2, grid=(4, 10), frames=5)
dev = torch.device("cuda:0"); bf = torch.bfloat16
rope = swk.Rope(w.n_heads, w.head_dim, w.dims, w.grid, w.theta0, w.sigma, None)
cache = swk.Cache(rope, 1, 1, 2, bf, device=dev)
outs = []
for f in range(w.frames):
    q, k, v = (torch.from_numpy(wl.frame_qkv(w, f, tensor=t)).to(dev, bf).contiguous()
               for t in (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
    swk.sa_cache_append(cache, k, v, 1, f)
    o = torch.empty_like(q)
    nbytes = swk.sa_window_attn_workspace(cache, 1)
    ws = torch.zeros(max(nbytes // 4, 4), dtype=torch.float32, device=dev)
    swk.sa_window_attn(cache, q, o, 1, 0.0, swk.SA_MASK_FRAME_CAUSAL, ws)
    outs.append(o.float().cpu().numpy())
n_res = 3
x = torch.randn(1, n_res * w.tokens_per_frame, 256, generator=torch.Generator().manual_seed(5)).to(dev, bf)
wk = (torch.randn(w.n_heads * w.head_dim, 256, generator=torch.Generator().manual_seed(6)) / 16).to(dev, bf)
wv = (torch.randn(w.n_heads * w.head_dim, 256, generator=torch.Generator().manual_seed(7)) / 16).to(dev, bf)
swk.sa_cache_recache(cache, x, wk, wv, 256)
for i in range(n_res):
    ko = torch.empty(1, w.tokens_per_frame, w.n_heads, w.head_dim, dtype=bf, device=dev)
    vo = torch.empty_like(ko)
    swk.sa_cache_read(cache, i, ko, vo)
    outs += [ko.float().cpu().numpy(), vo.float().cpu().numpy()]
torch.cuda.synchronize()
np.savez(sys.argv[2], *outs)
print("ok")
'''


def _run(tmp_path, name, debug):
    env = dict(os.environ)
    env.pop("SA_DEBUG_SYNC", None)
    if debug:
        env["SA_DEBUG_SYNC"] = "1"
    out = str(tmp_path / f"{name}.npz")
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT, out], env=env, capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0 and "ok" in r.stdout, f"{name}: rc {r.returncode}\n{r.stdout}\n{r.stderr[-2000:]}"
    d = np.load(out)
    return [d[k] for k in sorted(d.files, key=lambda s: int(s.split("_")[1]))]


def test_debug_sync_changes_no_result(tmp_path):
    plain = _run(tmp_path, "plain", False)
    synced = _run(tmp_path, "synced", True)
    assert len(plain) == len(synced) == 5 + 6
    for i, (a, b) in enumerate(zip(plain, synced)):
        assert np.isfinite(a).all()
        assert np.array_equal(a, b), f"output {i} differs with SA_DEBUG_SYNC=1"
