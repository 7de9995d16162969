"""OCP FP8 E5M2 codec in float64 (oracle; test infrastructure only).

The format of the MLP's gradients in modded-nanogpt ``gpt.py`` (FP8 MLP constants: the static
e5m2 scale of the incoming gradient, and the delayed dpre scale formed against the e5m2 maximum
57344, ``torch.finfo(torch.float8_e5m2).max``). Its definition (OCP 8-bit floating point
specification, E5M2):

* bit 7 sign, bits 6..2 exponent (bias 15), bits 1..0 mantissa;
* exponent field 0: subnormal, value 2^-14 * m/4 (smallest 2^-16);
* exponent field e in 1..30: value 2^(e-15) * (1 + m/4); the largest finite value is
  S.11110.11 = 57344;
* exponent field 31: infinity (mantissa 0) or NaN (mantissa != 0).

Encoding from a real value: round to the nearest representable value, ties to the code with an
even mantissa; magnitudes at or beyond 57344 saturate to +-57344 (the reading taken for the
e4m3 operands as well: a scaled tensor is meant to fit the range, and saturation keeps one
outlier from becoming an infinity); NaN maps to the NaN code 0x7F. The encoder is the plainest
form of that rule: a search of the 124 non-negative finite values.
"""
from __future__ import annotations

import numpy as np

E5M2_MAX = 57344.0
_NAN_CODE = 0x7F
_MAX_CODE = 0x7B      # S.11110.11


def e5m2_decode(codes) -> np.ndarray:
    """Value of each e5m2 code (uint8) as float64: infinities and NaNs as such."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 0x3).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 4.0, -14), np.ldexp(1.0 + m / 4.0, (e - 15).astype(np.int64)))
    mag = np.where(e == 0x1F, np.where(m == 0, np.inf, np.nan), mag)
    return s * mag


def e5m2_grid() -> np.ndarray:
    """The 124 non-negative finite values, indexed by their code 0x00..0x7B (increasing)."""
    return e5m2_decode(np.arange(0, _MAX_CODE + 1, dtype=np.uint8))


def e5m2_encode(values) -> np.ndarray:
    """Round real values (read exactly as float64) to e5m2 codes: nearest, ties to even
    mantissa, saturating at +-57344 (infinities too), NaN to 0x7F. Zero keeps its sign."""
    v = np.asarray(values, dtype=np.float64)
    grid = e5m2_grid()
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    finite = ~np.isnan(a)
    a_c = np.where(finite, np.minimum(a, E5M2_MAX), 0.0)
    hi = np.clip(np.searchsorted(grid, a_c, side="left"), 0, _MAX_CODE)   # grid[hi] >= a
    lo = np.clip(hi - 1, 0, _MAX_CODE)
    d_lo = a_c - grid[lo]
    d_hi = grid[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(grid[hi] == a_c, hi, np.where(pick_hi, hi, lo))
    code = np.where(finite, code, _NAN_CODE)
    return (code | sign).astype(np.uint8)
