"""Storage encoding of fp8 weights (OCP E4M3FN) used to *produce* the long-context workload's weights.

A Linear weight of that workload is stored as E4M3FN codes q[n, k] plus one float32 scale
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


def encode_e4m3fn_table(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even, saturating encode by search over the value table
    (slow; kept as the cross-check of :func:`encode_e4m3fn`)."""
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


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even, saturating encode of float64/float32 values.

    Codes are monotonic in magnitude, so the code of |x| is the rounded
    position of |x| on the E4M3FN grid: below 2^-6 the grid step is 2^-9
    (code = rint(|x| * 2^9)); in binade [2^e, 2^(e+1)) the step is 2^(e-3)
    and code = 8 (e + 7) + rint(|x| * 2^(3-e)) - 8. Scaling by a power of two
    is exact and ``rint`` rounds halves to even, which is the even-code rule
    (the code's parity is the parity of the rounded mantissa); a rounded
    mantissa of 16 carries into the next binade's first code by itself.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, ex = np.frexp(a)                         # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                  # binade exponent (the subnormal branch ignores it)
    sub = a < 2.0 ** -6
    q = np.rint(np.ldexp(a, np.where(sub, 9, 3 - e)))
    code = np.where(sub, q, 8.0 * (e + 7) + q - 8.0)
    mag = code.astype(np.uint8)
    sign = np.where(np.signbit(x) & (mag != 0), 0x80, 0x00).astype(np.uint8)
    return mag | sign


def quantize_rows(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-output-channel (row) scale and E4M3FN codes of a [N, K] weight."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1).astype(np.float64)
    scale = (amax / E4M3_MAX).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.empty(w.shape, dtype=np.uint8)
    step = max(1, (1 << 22) // max(1, w.shape[1]))     # rows per chunk: bounded float64 temporaries
    for r in range(0, w.shape[0], step):
        codes[r:r + step] = encode_e4m3fn(w[r:r + step].astype(np.float64) / scale[r:r + step].astype(np.float64)[:, None])
    return codes, scale
