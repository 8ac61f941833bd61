"""Device-side time-outs of the persistent DiT layer kernel, forced from the
host: the environment variable VLA_DIT_SPIN_LIMIT lowers the bound of the
kernel's own waits to one poll, so waits give up at once instead of hanging,
every workgroup leaves normally, and the pass must report VLA_ERR_TIMEOUT
through vla_workspace_status / vla_step_status with NaN outputs. The next
pass on the same workspace with the normal bound must be correct again (the
status word and the counters it left are cleared)."""

import numpy as np
import pytest

from oracle.policy import run_config
from synth import make_inputs, make_weights, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def test_dit_timeout_is_reported_and_the_next_pass_recovers(gu, monkeypatch):
    from vla_robot_policy_amd import lib
    cfg = small_config("dit", "bf16")
    W, I = make_weights(cfg), make_inputs(cfg)
    dw = gu.DeviceWeights(cfg, W)
    ws = gu.dit_workspace(cfg, dw)
    ctx, noise = gu.upload_input(I["ctx"]), gu.upload_input(I["noise"])
    monkeypatch.setenv("VLA_DIT_SPIN_LIMIT", "1")
    acts, vel = gu.run_dit(cfg, dw, ctx, noise, ws=ws)
    st = lib.vla_workspace_status(ws[0])
    gu.say(f"forced time-out: status {st}, NaN actions {np.isnan(acts).all()}")
    assert st == lib.VLA_ERR_TIMEOUT
    assert np.isnan(acts).all() and np.isnan(vel).all()
    monkeypatch.delenv("VLA_DIT_SPIN_LIMIT")
    acts, vel = gu.run_dit(cfg, dw, ctx, noise, ws=ws)
    assert lib.vla_workspace_status(ws[0]) == lib.VLA_OK
    want = run_config(cfg, W, I)
    gu.relerr(acts, want["actions"], 1e-2, "dit after a time-out, actions")
    gu.relerr(vel, want["velocities"], 1e-2, "dit after a time-out, velocities")


def test_step_timeout_is_reported_and_the_plan_recovers(gu, monkeypatch):
    from vla_robot_policy_amd import lib
    cfg = small_config("step", "bf16")
    W, I = make_weights(cfg), make_inputs(cfg)
    dw = gu.DeviceWeights(cfg, W)
    r = gu.StepRunner(cfg, dw, I)
    try:
        monkeypatch.setenv("VLA_DIT_SPIN_LIMIT", "1")
        r.run()
        bad = r.outputs()
        assert lib.vla_step_status(r.plan) == lib.VLA_ERR_TIMEOUT
        assert np.isnan(bad["actions"]).all()
        monkeypatch.delenv("VLA_DIT_SPIN_LIMIT")
        r.capture()                      # its warm-up pass, then the graph
        r.replay()
        got = r.outputs()
        assert lib.vla_step_status(r.plan) == lib.VLA_OK
        want = run_config(cfg, W, I)
        for k in ("hidden", "actions", "velocities"):
            gu.relerr(got[k], want[k], 1e-2, f"step after a time-out, {k}")
    finally:
        r.close()
