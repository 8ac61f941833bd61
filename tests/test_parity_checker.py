"""The parity checker's local (per-row) bar catches a single corrupted row
that the global bar lets through: a seq-130 block (two full 64-row tiles
and a ragged 2-row tail) evaluated by the oracle, with bf16-level noise on
every row and one row of the ragged tail off by 5 %."""

import numpy as np
import pytest

from oracle import llm
from oracle.io import Weights, to_f64
from synth import make_inputs, make_weights, small_config
from tests.parity import LOCAL_FACTOR, rel_errors, relerr


def _block_out():
    cfg = small_config("block", "bf16", seq=130)
    W, I = make_weights(cfg), make_inputs(cfg)
    return llm.block(to_f64(I["x"]), Weights(W), "llm.0.", cfg.block)


def test_one_corrupt_tail_row_fails_local_passes_global():
    want = _block_out()
    rng = np.random.default_rng(23)
    got = want * (1.0 + 2e-3 * rng.standard_normal(want.shape))    # bf16-level noise everywhere
    relerr(got, want, 1e-2, "noise only")                          # both bars hold
    bad = got.copy()
    bad[129] = want[129] * (1.0 + 0.05 * rng.standard_normal(want.shape[1]))   # the ragged tail's last row
    e, er, r = rel_errors(bad, want)
    assert e <= 1e-2 and r == 129 and er > LOCAL_FACTOR * 1e-2
    with pytest.raises(AssertionError, match="row 129"):
        relerr(bad, want, 1e-2, "planted row")


def test_global_bar_still_applies():
    want = _block_out()
    got = want * 1.02
    with pytest.raises(AssertionError, match="rel L2"):
        relerr(got, want, 1e-2, "uniform 2 %")


def test_rows_are_the_last_axis():
    want = np.ones((3, 4, 5))
    got = want.copy()
    got[1, 2] *= 1.5
    e, er, r = rel_errors(got, want)
    assert r == 1 * 4 + 2 and abs(er - 0.5) < 1e-12
