"""The parity measure of the GPU tests: relative L2 error against the oracle,
per tensor and per row.

A tensor's error is ||got - want||_2 / ||want||_2 over all its elements
(the tolerance the workloads are graded on: 1e-2 for bf16, 5e-2 for 8-bit
weights). A single wrong row of a 100-row tensor moves that global figure
by only about a tenth of its own error, so the check is also local: every
row (a token of a hidden state, a row of an action chunk; the last axis is
the row) must be within LOCAL_FACTOR times the tensor's bar on its own.
"""

from __future__ import annotations

import numpy as np

LOCAL_FACTOR = 3.0


def rel_errors(got, want):
    """(global relative L2 error, worst per-row relative L2 error, its row)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    e = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    g2 = got.reshape(-1, got.shape[-1]) if got.ndim > 1 else got.reshape(1, -1)
    w2 = want.reshape(g2.shape)
    den = np.linalg.norm(w2, axis=1)
    num = np.linalg.norm(g2 - w2, axis=1)
    live = den > 0
    rows = np.where(live, num / np.where(live, den, 1.0), np.where(num > 0, np.inf, 0.0))
    worst = int(np.argmax(rows))
    return e, float(rows[worst]), worst


def relerr(got, want, bar=None, label: str = "") -> float:
    """Global relative L2 error of got against want. With a bar, also assert
    it (global <= bar, every row <= LOCAL_FACTOR * bar) and print both."""
    e, er, r = rel_errors(got, want)
    if bar is not None:
        print(f"  parity {label}: rel L2 {e:.3e} (bar {bar:.0e}), worst row {r}: {er:.3e} "
              f"(bar {LOCAL_FACTOR * bar:.0e})", flush=True)
        assert e <= bar, f"{label}: rel L2 {e:.3e} > {bar}"
        assert er <= LOCAL_FACTOR * bar, f"{label}: row {r} rel L2 {er:.3e} > {LOCAL_FACTOR * bar}"
    return e
