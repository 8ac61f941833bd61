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
