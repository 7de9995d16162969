"""OCP FP8 E4M3 ("e4m3fn") codec in float64 (oracle; test infrastructure only).

The format is the one modded-nanogpt ``gpt.py`` quantizes its MLP operands to
(``torch.float8_e4m3fn``, whose finite maximum 448 its FP8 constants and
``_quantize_mlp_weights_and_scales`` divide by). Its definition (OCP 8-bit floating point
specification, E4M3):

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent field 0: subnormal, value 2^-6 * m/8 (smallest 2^-9);
* exponent field e > 0: value 2^(e-7) * (1 + m/8);
* S.1111.111 is NaN; there is no infinity, so the largest finite value is S.1111.110 = 448.

Encoding from a real value: round to the nearest representable value, ties to the code with an
even mantissa; magnitudes at or beyond 448 saturate to +-448 (the page notes that e4m3 with a
static scale "saturates entries beyond" its range); NaN maps to NaN. The encoder below is the
plainest form of that rule: a search of the 127 non-negative finite values.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F
_MAX_CODE = 0x7E


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 code (uint8) as float64; NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return s * mag


def e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite values, indexed by their code 0x00..0x7E (increasing)."""
    return e4m3_decode(np.arange(0, _MAX_CODE + 1, dtype=np.uint8))


def e4m3_encode(values) -> np.ndarray:
    """Round real values (read exactly as float64) to e4m3 codes: nearest, ties to even
    mantissa, saturating at +-448, NaN to the NaN code. The sign bit is kept for zero."""
    v = np.asarray(values, dtype=np.float64)
    grid = e4m3_grid()
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    finite = ~np.isnan(a)
    a_c = np.where(finite, np.minimum(a, E4M3_MAX), 0.0)
    hi = np.clip(np.searchsorted(grid, a_c, side="left"), 0, _MAX_CODE)   # grid[hi] >= a
    lo = np.clip(hi - 1, 0, _MAX_CODE)
    d_lo = a_c - grid[lo]
    d_hi = grid[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(grid[hi] == a_c, hi, np.where(pick_hi, hi, lo))
    code = np.where(finite, code, _NAN_CODE)
    return (code | sign).astype(np.uint8)
