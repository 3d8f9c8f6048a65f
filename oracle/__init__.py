"""CPU oracle for the frame-sink + short-window KV attention path (fp64 numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never calls it and shares no code with it; the only thing the two
sides share is the seeded input generator in ``workloads``.

Every function is the plain definition of what the method computes, in
float64, written from the pages:

* ``rope``      -- per-head jittered bases and frequencies, 3D RoPE rotation
                   (LoL paper review, background "Rotary Position Embedding"
                   rotation matrix; "method steps" (2)-(7)).
* ``cache``     -- which frames are resident and in which slot: pinned sink
                   frames plus a sliding local window (LongLive paper review,
                   section 3 "Frame Sink", section 6 table "attention window").
* ``attention`` -- softmax(q k^T / sqrt(d)) v over the resident frames
                   (LongLive paper review, section 3 "Short-Window Attention"
                   equation; LoL paper review, background "multi-head
                   attention" equation).
* ``recache``   -- K, V = x W_k, x W_v over the cached frames, K re-rotated
                   (LongLive paper review, section 3 "KV Recache").
* ``project``   -- per-frame q, k, v = x W_q, x W_k, x W_v with (k, v)
                   appended to the cache, and a plain linear map x W
                   (LoL paper review, background "multi-head attention";
                   LongLive paper review, section 3 "KV Recache").
* ``diagnostics`` -- per-head softmax mass on the sink frames and the
                   phase-coherence kernel C(Delta) (LoL paper review, "core
                   method" and "core innovation" paragraphs).
* ``fp8``       -- e4m3 rounding of the FP8 cache (OCP 8-bit float, the
                   format the reviewed model card's FP8 variant is read as).
* ``quant``     -- row-wise 8-bit quantisation (int8, e4m3) and the W8A8
                   product of the 8-bit projections (LongLive paper review,
                   "INT8 quantized inference" table; model card FP8 variant).
* ``brute``     -- pure-Python loop versions for tiny shapes, used to pin the
                   numpy versions.
* ``stream``    -- composes the above into the per-frame stream the library
                   runs (append, then attend).

Pins (tests/test_oracle_*.py) tie these to closed forms, invariants,
library routines and brute force; see the test docstrings.
"""
from . import rope, cache, attention, recache, project, brute, stream, diagnostics, fp8, quant  # noqa: F401
