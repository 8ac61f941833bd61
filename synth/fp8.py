"""Storage encoding of fp8 weights (OCP E4M3FN) used to *produce* the cfg5 inputs.

A cfg5 Linear weight is stored as E4M3FN codes q[n, k] plus one float32 scale
s[n] per output channel, s[n] = max_k |W[n, k]| / 448 (448 is the largest
finite E4M3FN magnitude). q is W/s rounded to the nearest E4M3FN value, ties
to the value whose code is even, saturating at +-448. The (q, s) pair is the
model weight both the oracle and the GPU path consume; how a consumer turns a
code back into a number is not defined here.

E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
subnormal (m/8 * 2^-6); the codes 0x7F and 0xFF are NaN; there is no infinity.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _nonneg_table() -> tuple[np.ndarray, np.ndarray]:
    """All finite non-negative E4M3FN values (ascending) and their codes."""
    vals, codes = [], []
    for code in range(0x00, 0x7F):          # 0x7F is NaN
        e, m = (code >> 3) & 0xF, code & 0x7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(v)
        codes.append(code)
    return np.asarray(vals, dtype=np.float64), np.asarray(codes, dtype=np.uint8)


_VALS, _CODES = _nonneg_table()


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even, saturating encode of float64/float32 values."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_VALS, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, len(_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_VALS) - 1)
    d_hi = _VALS[hi] - a
    d_lo = a - _VALS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_CODES[hi] & 1) == 0))
    mag = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.uint8)
    sign = np.where(np.signbit(x) & (mag != 0), 0x80, 0x00).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def quantize_rows(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-output-channel (row) scale and E4M3FN codes of a [N, K] weight."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1).astype(np.float64)
    scale = (amax / E4M3_MAX).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = encode_e4m3fn(w.astype(np.float64) / scale.astype(np.float64)[:, None])
    return codes, scale
