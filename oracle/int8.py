"""INT8 activations of the W8A8 integer variant (oracle side).

Page "开源 APXInf 把 VLA 推理压到 26 毫秒" (section on CUDA Graph, FP8 and Rust):
on hardware without FP8 units the runtime quantises to INT8 instead. Plain
reading where the page is silent, the integer counterpart of the FP8 rule in
oracle/fp8.py: each activation row (token) gets its own scale at run time,
s = max|x| / 127, and x / s is rounded to the nearest integer (halves to
even) and clipped to [-127, 127]. The decision is taken in float32, the
precision the kernels compute it in: x * (127 / max|x|) is one float32
multiply by a float32 reciprocal.
"""

from __future__ import annotations

import numpy as np


def quantize_act_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row int8 codes and float32 scales of activations x [M, K]."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=1)
    inv = np.where(amax > 0, np.float32(127.0) / np.where(amax > 0, amax, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    y = (x32 * inv[:, None]).astype(np.float32)
    codes = np.clip(np.rint(y), -127, 127).astype(np.int8)
    return codes, (amax / np.float32(127.0)).astype(np.float32)


def fake_quant_act_rows(x: np.ndarray) -> np.ndarray:
    """The values W8A8 integer GEMMs see for activations x: codes times row scale."""
    codes, scale = quantize_act_rows(x)
    return codes.astype(np.float64) * scale.astype(np.float64)[:, None]
