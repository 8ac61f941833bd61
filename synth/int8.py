"""Storage encoding of int8 weights used to *produce* the int8 workload's weights.

An int8 Linear weight is stored as codes q[n, k] in [-127, 127] plus one
float32 scale s[n] per output channel, s[n] = max_k |W[n, k]| / 127; q is
W / s rounded to the nearest integer (halves to even). The (q, s) pair is
the model weight both the oracle and the GPU path consume.
"""

from __future__ import annotations

import numpy as np


def quantize_rows(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-output-channel (row) scale and int8 codes of a [N, K] weight."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1).astype(np.float64)
    scale = (amax / 127.0).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(w.astype(np.float64) / scale.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    return codes, scale
