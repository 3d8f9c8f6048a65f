"""Helpers for the GPU parity tests: tolerances, metrics and stream drivers.

Tolerances: bf16 paths rel-L2 <= 5e-3 and max-abs <= 2e-2 against the fp64
oracle; fp32 paths <= 1e-5 on both.
"""
from __future__ import annotations

import contextlib
import sys

import numpy as np

BF16_REL, BF16_ABS = 5e-3, 2e-2
F32_REL, F32_ABS = 1e-5, 1e-5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(got - ref).max()) if got.size else 0.0
    return rel, mx


def assert_close(got, ref, dtype: str, what: str):
    rel, mx = metrics(got, ref)
    r_tol, a_tol = (BF16_REL, BF16_ABS) if dtype == "bf16" else (F32_REL, F32_ABS)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert rel <= r_tol and mx <= a_tol, f"{what}: rel_l2 {rel:.3e} (tol {r_tol}), max_abs {mx:.3e} (tol {a_tol})"
    return rel, mx


def to_dev(a, dtype_str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16 if dtype_str == "bf16" else torch.float32).contiguous()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def torch_dtype(dtype_str):
    import torch
    return torch.bfloat16 if dtype_str == "bf16" else torch.float32


def sample_rows(L: int, T: int, n: int = 160, seed: int = 0):
    """Rows to check at large sizes: both ends of every frame, the ragged tail and random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for f in range(L // T):
        for r in (0, 1, 31, 32, 127, 128, T - 25, T - 24, T - 1):
            if 0 <= r < T:
                rows.add(f * T + r)
    rows.update(rng.integers(0, L, size=n).tolist())
    return np.array(sorted(rows))


_KNOBS = {"kernel": 0, "splits": 1, "tile": 2}


@contextlib.contextmanager
def launch_override(kernel=None, splits=None, tile=None):
    """Force the bf16 attention kernel variant / key splits / projection tile (sa_set_launch_override)
    for the block.

    None leaves a knob automatic; tile counts from 0 (256 x 128, 128 x 128, 128 x 64, 256 x 256).
    """
    import sink_window_kv_amd as swk
    vals = {"kernel": kernel, "splits": splits, "tile": None if tile is None else int(tile) + 1}
    for k, v in vals.items():
        swk.sa_set_launch_override(_KNOBS[k], 0 if v is None else int(v))
    try:
        yield
    finally:
        for k in vals:
            swk.sa_set_launch_override(_KNOBS[k], 0)
