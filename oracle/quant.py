"""Oracle: 8-bit projections -- row-wise quantisation and the W8A8 product.

Test infrastructure only (see ``oracle/__init__``).

Sources:
* LongLive paper review, "INT8 quantized inference" table: the INT8 model
  halves the model size and raises throughput with little quality loss
  (12.6 -> 16.4 FPS); no scheme is given.
* LongLive model card (abstract): an FP8 variant (24.8 FPS); no format or
  scaling given.

Readings taken (the pages fix none of this):
* W8A8: both operands of a projection are 8-bit codes with one fp32 scale
  per row -- per token for the activations x [n][C], per output feature for
  the weights W [F][C] -- so y[n][f] = sx[n] sw[f] sum_c qx[n][c] qw[f][c].
  Codes are int8 (symmetric, |q| <= 127) or OCP e4m3 (|q| <= 448, see
  ``fp8``).
* A row is quantised from its largest magnitude a: s = a / Q with Q = 127
  (int8) or 448 (e4m3), codes = round(x * (Q / a)), nearest with ties to
  even, clamped to +-Q; a row of zeros gets s = 0 and codes 0.  These
  decisions are taken in fp32 (the precision of the kernels), step by step
  as written: a, Q / a, x * (Q / a), the rounding, and a / Q.
* For int8 the integer sum is exact; the output is taken in fp32 as
  (float(acc) * sx[n]) * sw[f] and rounded to bf16 (nearest even).  For
  e4m3 the output is the exact product of the decoded values times the two
  scales, in fp64.
"""
from __future__ import annotations

import numpy as np

from . import fp8 as _fp8

QMAX = {"int8": 127.0, "e4m3": 448.0}


def e4m3_encode(v) -> np.ndarray:
    """Byte code of values that are exactly representable in e4m3 (sign kept for zeros)."""
    v = np.asarray(v, dtype=np.float64)
    table = _fp8.decode(np.arange(0x7F))            # magnitudes of codes 0x00 .. 0x7e, increasing
    mag = np.searchsorted(table, np.abs(v))
    if not np.all(table[np.minimum(mag, 0x7E)] == np.abs(v)):
        raise ValueError("value not representable in e4m3")
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows(x, qtype: str):
    """Row-wise quantisation of x [n][C] (values exactly representable in fp32).

    Returns (codes [n][C]: int8 or uint8 e4m3 bytes, scales [n] float32).
    """
    x32 = np.asarray(x, dtype=np.float32)
    q = np.float32(QMAX[qtype])
    amax = np.max(np.abs(x32), axis=1)                       # fp32, exact
    nz = amax > 0
    inv = np.zeros_like(amax)
    inv[nz] = q / amax[nz]                                  # fp32 division
    y = x32 * inv[:, None]                                  # fp32 product
    scales = np.zeros_like(amax)
    scales[nz] = amax[nz] / q                               # fp32 division
    if qtype == "int8":
        codes = np.clip(np.rint(y), -127, 127).astype(np.int8)   # rint: ties to even
    else:
        codes = e4m3_encode(_fp8.round_e4m3(np.clip(y.astype(np.float64), -448.0, 448.0)))
    return codes, scales


def decode(codes, qtype: str) -> np.ndarray:
    """Code values in float64 (int8 as integers, e4m3 from the bit fields)."""
    if qtype == "int8":
        return np.asarray(codes, dtype=np.int8).astype(np.float64)
    return _fp8.decode(np.asarray(codes, dtype=np.uint8))


def dequantize(codes, scales, qtype: str) -> np.ndarray:
    """s_row * value(code), float64 [n][C]."""
    return np.asarray(scales, dtype=np.float64)[:, None] * decode(codes, qtype)


def linear_q8(cx, sx, cw, sw, qtype: str) -> np.ndarray:
    """y [n][F] = sx[n] sw[f] sum_c qx[n][c] qw[f][c] (codes cx [n][C], cw [F][C]).

    int8: exact integer sums, then (float32(acc) * sx) * sw in fp32 (returned as
    float32, before the bf16 rounding).  e4m3: float64.
    """
    if qtype == "int8":
        acc = np.asarray(cx, dtype=np.int64) @ np.asarray(cw, dtype=np.int64).T
        sx32 = np.asarray(sx, dtype=np.float32)[:, None]
        sw32 = np.asarray(sw, dtype=np.float32)[None, :]
        return (acc.astype(np.float32) * sx32) * sw32
    acc = decode(cx, qtype) @ decode(cw, qtype).T
    return acc * np.asarray(sx, dtype=np.float64)[:, None] * np.asarray(sw, dtype=np.float64)[None, :]
