"""V-AEFusion plans on the GPU (page "跨XPU平台表征视觉-语言-动作模型：机器人部署中
的约束与加速", section 5.3): every pass is one control cycle whose first
n_stale Euler steps cross-attend to the previous cycle's context while the
VLM of the cycle runs on another stream (or graph branch).

The configuration pairs a small vision encoder and backbone with a DiT of the
full width (1280), so the action branch runs the persistent layer kernel
alongside the VLM kernels. Three cycles on fresh inputs each are checked
against the float64 oracle's cycle chain; a captured plan must reproduce the
eager cycles bit for bit; with no stale step a fused plan must reproduce the
plain plan bit for bit."""

import dataclasses

import numpy as np
import pytest

from oracle.io import Weights, to_f64
from oracle.policy import vla_cycle_fused
from synth import make_inputs, make_weights, small_config
from synth.configs import DiTShape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _cfg():
    return small_config("step", "bf16", dit=DiTShape(layers=2), steps=4)


def _inputs(cfg, n):
    return [make_inputs(cfg.replace(cid=cfg.cid + i)) for i in range(n)]


def _args(I):
    return to_f64(I["image"]), to_f64(I["text"]), to_f64(I["noise"])


@pytest.fixture(scope="module")
def setup(gu):
    cfg = _cfg()
    W = make_weights(cfg)
    return cfg, W, gu.DeviceWeights(cfg, W), _inputs(cfg, 3)


def test_fused_cycles_against_the_oracle_chain(gu, setup):
    from vla_robot_policy_amd import lib
    cfg, W, dw, ins = setup
    Wo = Weights(W)
    n_stale = 2
    r = gu.StepRunner(cfg, dw, ins[0], n_stale=n_stale)
    eager, prev = [], None
    try:
        for c, I in enumerate(ins):
            r.load(I)
            r.run()
            got = r.outputs()
            want = vla_cycle_fused(*_args(I), prev, Wo, cfg, n_stale)
            prev = want["ctx"]
            for k in ("hidden", "actions", "velocities"):
                e = gu.relerr(got[k], want[k], gu.TOL["bf16"], f"fused cycle {c} {k}")
                assert e <= gu.TOL["bf16"], (c, k, e)
            eager.append(got)
        assert lib.vla_step_cycles(r.plan) == 3
    finally:
        r.close()
    # the same cycles from graphs: capture runs cycle 0, replays run 1 and 2
    g = gu.StepRunner(cfg, dw, ins[0], n_stale=n_stale)
    try:
        g.capture()
        got = g.outputs()
        for k in got:
            assert np.array_equal(got[k], eager[0][k]), ("cycle 0", k)
        assert lib.vla_step_graph_nodes(g.plan) > 0
        for c in (1, 2):
            g.load(ins[c])
            g.replay()
            got = g.outputs()
            for k in got:
                assert np.array_equal(got[k], eager[c][k]), (c, k)
        assert lib.vla_step_cycles(g.plan) == 3
        assert lib.vla_step_run_shape(g.plan, g.shape) == lib.VLA_ERR_UNSUPPORTED
    finally:
        g.close()


def test_fused_without_stale_steps_is_the_plain_step(gu, setup):
    cfg, W, dw, ins = setup
    p = gu.StepRunner(cfg, dw, ins[1])
    f = gu.StepRunner(cfg, dw, ins[0], n_stale=0)
    try:
        p.run()
        plain = p.outputs()
        f.capture()           # cycle 0 on ins[0]
        f.load(ins[1])
        f.replay()            # cycle 1: no stale step, so the plain step on ins[1]
        got = f.outputs()
        for k in got:
            assert np.array_equal(got[k], plain[k]), k
    finally:
        p.close()
        f.close()


def test_fused_unchanged_observation_is_the_plain_step(gu, setup):
    """Stale steps on a context equal to the current one change nothing."""
    cfg, W, dw, ins = setup
    p = gu.StepRunner(cfg, dw, ins[2])
    f = gu.StepRunner(cfg, dw, ins[2], n_stale=cfg.steps)
    try:
        p.run()
        plain = p.outputs()
        f.capture()           # cycle 0
        for _ in range(2):    # cycles 1, 2: every step stale, on the same observation
            f.replay()
            got = f.outputs()
            for k in got:
                assert np.array_equal(got[k], plain[k]), k
    finally:
        p.close()
        f.close()
