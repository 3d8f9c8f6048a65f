"""Build libsinkattn.so in-tree with hipcc for gfx950.

Usage: python -m sink_window_kv_amd.build  (or __graft_entry__.build()).
Objects go to sink_window_kv_amd/_build/, the library to
sink_window_kv_amd/libsinkattn.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsinkattn.so")
SOURCES = ["api.cpp", "rope_append.hip", "window_attn.hip", "window_attn_fp8.hip", "proj_gemm.hip", "quantize.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep matrix-core accumulators in ordinary VGPRs where they fit (avoids
    # AGPR<->VGPR copies around the softmax, which reads the score tiles)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-inline-asm",  # the LDS-DMA asm names m0, which it sets itself
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# Per-source extra flags.  The attention kernel never sees a NaN (masked
# scores are -inf, every finite input stays finite), so NaN-aware max/min
# canonicalisation is dropped there.
EXTRA = {"window_attn.hip": ["-fno-honor-nans"], "window_attn_fp8.hip": ["-fno-honor-nans"]}


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
