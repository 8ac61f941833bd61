"""Pins of the V-AEFusion sampler and cycle (page "跨XPU平台表征视觉-语言-动作模型：
机器人部署中的约束与加速", section 5.3): the first n_stale Euler steps of a
cycle are conditioned on the previous cycle's context, the rest on the
current one. Checked against the plain sampler in its limiting cases, the
Euler scheme's own invariants, and the velocity field at the switch."""

import numpy as np
import pytest

from oracle import dit, policy
from oracle.io import Weights, to_f64
from synth import make_inputs, make_weights, small_config


@pytest.fixture(scope="module")
def setup():
    cfg = small_config("dit", "bf16")
    W = Weights(make_weights(cfg))
    cur, prev = make_inputs(cfg), make_inputs(small_config("dit", "bf16", seed=1001))
    return cfg, W, to_f64(cur["noise"]), to_f64(prev["ctx"]), to_f64(cur["ctx"])


def _plain(cfg, W, noise, ctx):
    rec = []
    a = dit.flow_sample(noise, ctx, W, cfg.dit, cfg.steps, rec)
    return a, rec


def _stale(cfg, W, noise, prev, cur, s):
    rec = []
    a = dit.flow_sample_stale(noise, prev, cur, W, cfg.dit, cfg.steps, s, rec)
    return a, rec


def test_no_stale_step_is_the_plain_sampler(setup):
    cfg, W, noise, prev, cur = setup
    a, rec = _stale(cfg, W, noise, prev, cur, 0)
    b, rb = _plain(cfg, W, noise, cur)
    assert np.array_equal(a, b)
    assert all(np.array_equal(x, y) for x, y in zip(rec, rb))


def test_all_stale_steps_is_the_plain_sampler_on_the_previous_context(setup):
    cfg, W, noise, prev, cur = setup
    a, _ = _stale(cfg, W, noise, prev, cur, cfg.steps)
    b, _ = _plain(cfg, W, noise, prev)
    assert np.array_equal(a, b)


def test_unchanged_observation_makes_staleness_harmless(setup):
    cfg, W, noise, prev, cur = setup
    b, _ = _plain(cfg, W, noise, cur)
    for s in range(cfg.steps + 1):
        a, _ = _stale(cfg, W, noise, cur, cur, s)
        assert np.array_equal(a, b), s


@pytest.mark.parametrize("s", [1, 2])
def test_switch_happens_after_exactly_n_stale_steps(setup, s):
    cfg, W, noise, prev, cur = setup
    K = cfg.steps
    assert 0 < s < K
    a, rec = _stale(cfg, W, noise, prev, cur, s)
    _, rp = _plain(cfg, W, noise, prev)
    # the stale prefix is the previous context's trajectory, step for step
    for k in range(s):
        assert np.array_equal(rec[k], rp[k]), k
    # the first fresh step is the velocity field under the current context
    # at the state the prefix reached, at time s / K
    x_s = noise + np.sum(rp[:s], axis=0) / K
    v = dit.dit_velocity(x_s, s / K, cur, W, cfg.dit)
    np.testing.assert_allclose(rec[s], v, rtol=1e-12, atol=1e-12)
    assert not np.allclose(rec[s], rp[s], rtol=1e-3)          # the conditioning did change
    # Euler: the result is the noise plus the mean of the recorded velocities
    np.testing.assert_allclose(a, noise + np.sum(rec, axis=0) / K, rtol=1e-12, atol=1e-12)


def test_n_stale_outside_the_step_range_is_rejected(setup):
    cfg, W, noise, prev, cur = setup
    for s in (-1, cfg.steps + 1):
        with pytest.raises(ValueError):
            dit.flow_sample_stale(noise, prev, cur, W, cfg.dit, cfg.steps, s)


def test_fused_cycle_chain():
    """Two cycles: the first has no previous context and equals the plain
    step; the second conditions its stale steps on the first cycle's context
    and leaves the VLM outputs untouched."""
    cfg = small_config("step", "bf16")
    W = Weights(make_weights(cfg))
    I0, I1 = make_inputs(cfg), make_inputs(small_config("step", "bf16", seed=1001))
    args = lambda I: (to_f64(I["image"]), to_f64(I["text"]), to_f64(I["noise"]))
    c0 = policy.vla_cycle_fused(*args(I0), None, W, cfg, 2)
    p0 = policy.vla_step(*args(I0), W, cfg)
    assert np.array_equal(c0["actions"], p0["actions"])
    c1 = policy.vla_cycle_fused(*args(I1), c0["ctx"], W, cfg, 2)
    p1 = policy.vla_step(*args(I1), W, cfg)
    for k in ("hidden", "ctx"):
        assert np.array_equal(c1[k], p1[k]), k
    rec = []
    want = dit.flow_sample_stale(to_f64(I1["noise"]), c0["ctx"], p1["ctx"], W, cfg.dit, cfg.steps, 2, rec)
    assert np.array_equal(c1["actions"], want)
    assert not np.allclose(c1["actions"], p1["actions"], rtol=1e-3)
