"""OCP E4M3FN decoding and per-output-channel dequantisation (oracle side).

Format (OCP 8-bit floating point specification, E4M3 "FN" variant): sign bit
7, exponent bits 6..3 with bias 7, mantissa bits 2..0. Exponent field 0 is
subnormal, value (m/8) * 2^-6; otherwise (1 + m/8) * 2^(e-7). Exponent 15
with mantissa 7 (codes 0x7F, 0xFF) is NaN; there are no infinities, so the
largest finite magnitude is 1.75 * 2^8 = 448.

The fp8 weights of the long-context workload follow the APXInf report's FP8
weight storage (page "开源 APXInf 把 VLA 推理压到 26 毫秒", section on CUDA
Graph, FP8 and Rust): a Linear weight is codes q[n, k] and a float32 scale
s[n] per output channel, and the weight it stands for is q * s.
"""

from __future__ import annotations

import numpy as np


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = sign * np.where(e == 0, sub, nor)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


# the 256 code values, from the definition above (a weight decodes by lookup)
_TABLE = decode_e4m3fn(np.arange(256))


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)[:, None]


# ---------------------------------------------------------------- activations
# W8A8 (page "开源 APXInf 把 VLA 推理压到 26 毫秒", same section: FP8 applied to
# the weights and the activations). Plain reading where the page is silent:
# each activation row (token) gets its own scale at run time, s = max|x| / 448,
# and x / s is rounded to the nearest E4M3FN value (ties to the even code,
# saturating at 448). The decision is taken in float32, the precision the
# kernels compute it in: x and max|x| are float32 values, x * (448 / max|x|)
# is one float32 multiply by a float32 reciprocal.

_FINITE = _TABLE[:0x7F]                       # non-negative finite values, ascending, codes 0x00..0x7E


def encode_e4m3fn_nearest(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of each value by search over the decoded table
    (ties to the even code, saturating at +-448). The sign bit is the
    value's, so a negative value that rounds to zero is -0 (0x80), as in
    IEEE rounding; the page does not say, and both zeros decode to 0."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 448.0)
    hi = np.clip(np.searchsorted(_FINITE, a, side="left"), 0, len(_FINITE) - 1)
    lo = np.clip(hi - 1, 0, len(_FINITE) - 1)
    d_hi, d_lo = _FINITE[hi] - a, a - _FINITE[lo]
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_act_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3FN codes and float32 scales of activations x [M, K]."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=1)
    inv = np.where(amax > 0, np.float32(448.0) / np.where(amax > 0, amax, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    y = (x32 * inv[:, None]).astype(np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    return encode_e4m3fn_nearest(y), scale


def fake_quant_act_rows(x: np.ndarray) -> np.ndarray:
    """The values W8A8 GEMMs see for activations x: codes times row scale."""
    codes, scale = quantize_act_rows(x)
    return dequantize_rows(codes, scale)

