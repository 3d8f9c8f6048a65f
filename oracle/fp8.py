"""Oracle: e4m3 (OCP 8-bit float) rounding for the FP8 cache (fp64).

Test infrastructure only (see ``oracle/__init__``).

Source: the LongLive model card and abstract report an FP8 variant of the
model (no format or scaling given).

Readings taken:
* FP8 is OCP e4m3 ("E4M3FN"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals (exponent field 0) of step 2^-9, largest
  finite magnitude 448 (0x7e), no infinities.  Rounding is to nearest,
  ties to even.
* A cache in FP8 stores rotated keys as e4m3(k / k_scale) and values as
  e4m3(v / v_scale) with one scale per tensor, values clamped to +-448
  before rounding; attention reads k_scale * key and v_scale * value.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


def decode(code) -> np.ndarray:
    """Value of e4m3 byte(s), from the bit fields; NaN for 0x7f / 0xff."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def round_e4m3(x) -> np.ndarray:
    """Nearest e4m3 value of x (ties to even), after clamping to +-448."""
    x = np.clip(np.asarray(x, dtype=np.float64), -MAX, MAX)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # exponent of the binade; subnormals share 2^-6
    ulp = np.exp2(e - 3.0)                    # 3 mantissa bits
    r = np.round(a / ulp) * ulp               # numpy rounds half to even
    return np.sign(x) * np.minimum(r, MAX)


def quantize(x, scale: float) -> np.ndarray:
    """What an FP8 cache gives back for x stored with `scale`: scale * e4m3(x / scale)."""
    return scale * round_e4m3(np.asarray(x, dtype=np.float64) / scale)
