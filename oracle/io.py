"""Float64 views of the stored seeded tensors (oracle side).

A stored tensor is float32, bfloat16 bits (uint16: the value is the float32
whose upper 16 bits are these and lower 16 bits are zero) or E4M3FN codes
with a per-row scale. The oracle always computes on the exact stored values,
upcast to float64, so weight rounding is not part of any error budget.
"""

from __future__ import annotations

import numpy as np

from .fp8 import dequantize_rows


def to_f64(t) -> np.ndarray:
    if t.dtype == "f32":
        return np.asarray(t.data, dtype=np.float64)
    if t.dtype == "bf16":
        u = np.asarray(t.data, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if t.dtype == "fp8":
        return dequantize_rows(t.data, t.scale)
    if t.dtype == "int8":   # integer codes times the row's scale
        return np.asarray(t.data, dtype=np.float64) * np.asarray(t.scale, dtype=np.float64)[:, None]
    raise ValueError(t.dtype)


class Weights:
    """Name -> float64 array over a ``synth`` TensorSet (converted per access)."""

    def __init__(self, tensors, keep: bool = False):
        self.t = tensors
        self.keep = keep
        self._c = {}

    def __getitem__(self, name: str) -> np.ndarray:
        if name in self._c:
            return self._c[name]
        v = to_f64(self.t[name])
        if self.keep:
            self._c[name] = v
        return v

    def __contains__(self, name: str) -> bool:
        return name in self.t
