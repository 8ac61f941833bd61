"""Helpers of the GPU parity tests: run the HIP path on seeded inputs through
the C ABI and compare with the oracle."""

from __future__ import annotations

import ctypes as C
import sys
import time

import numpy as np
import torch

from oracle.io import Weights
from tests.parity import relerr  # noqa: F401  (global and per-row bars)
from synth import make_inputs, make_weights
from vla_robot_policy_amd import lib
from vla_robot_policy_amd.device import DeviceWeights, bf16_bits_to_float, upload_input, workspace

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2, "int8": 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()




def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return t.detach().cpu().numpy().astype(np.float64)
    return bf16_bits_to_float(t).astype(np.float64)


def act_dtype(cfg) -> str:
    return "f32" if cfg.wdtype == "f32" else "bf16"


def act_empty(cfg, shape):
    return torch.empty(shape, dtype=torch.float32 if cfg.wdtype == "f32" else torch.int16, device=DEV)


def run_block(cfg, dw: DeviceWeights, x_in: torch.Tensor, seq: int) -> np.ndarray:
    bb = dw.backbone if dw.backbone is not None else dw.build_backbone()
    out = act_empty(cfg, (seq, cfg.block.hidden))
    need = lib.vla_block_workspace_bytes(dw.block_cfg, seq)
    ws = workspace(need)
    lib.check(lib.vla_block_forward(dw.block_cfg, bb.layers[0], x_in, out, seq, ws, need))
    torch.cuda.synchronize()
    return to_host(out, act_dtype(cfg))


def run_backbone(cfg, dw: DeviceWeights, e_in: torch.Tensor, seq: int) -> np.ndarray:
    bb = dw.backbone if dw.backbone is not None else dw.build_backbone()
    out = act_empty(cfg, (seq, cfg.block.hidden))
    need = lib.vla_backbone_workspace_bytes(bb, seq)
    ws = workspace(need)
    lib.check(lib.vla_backbone_prefill(bb, e_in, seq, out, ws, need))
    torch.cuda.synchronize()
    return to_host(out, act_dtype(cfg))


def dit_workspace(cfg, dw: DeviceWeights, ctx_len=None, K=None):
    dit = dw.dit if dw.dit is not None else dw.build_dit()
    d = cfg.dit
    need = lib.vla_dit_workspace_bytes(dit, cfg.ctx_len if ctx_len is None else ctx_len, d.chunk, d.action_dim,
                                       cfg.steps if K is None else K)
    return workspace(need), need


def run_dit(cfg, dw: DeviceWeights, ctx: torch.Tensor, noise: torch.Tensor, ctx_len=None, K=None, ws=None):
    """The Euler sampler through vla_flow_euler_sample; `ws` = (buffer, bytes)
    to run on a given workspace (default: a fresh one)."""
    d = cfg.dit
    dit = dw.dit if dw.dit is not None else dw.build_dit()
    ctx_len = cfg.ctx_len if ctx_len is None else ctx_len
    K = cfg.steps if K is None else K
    n, A = noise.shape
    acts = torch.empty((n, A), dtype=torch.float32, device=DEV)
    vel = torch.empty((K, n, A), dtype=torch.float32, device=DEV)
    if ws is None:
        need = lib.vla_dit_workspace_bytes(dit, ctx_len, n, A, K)
        ws = (workspace(need), need)
    lib.check(lib.vla_flow_euler_sample(dit, ctx, ctx_len, noise, n, A, K, acts, vel, ws[0], ws[1]))
    torch.cuda.synchronize()
    return acts.cpu().numpy().astype(np.float64), vel.cpu().numpy().astype(np.float64)


class StepRunner:
    """A vla_step plan over static device I/O buffers."""

    def __init__(self, cfg, dw: DeviceWeights, inputs, with_hidden=True, n_stale=None):
        self.cfg = cfg
        self.dw = dw
        model = dw.model if dw.model is not None else dw.build_model()
        d = cfg.dit
        self.images = upload_input(inputs["image"]) if cfg.vit is not None else None
        self.text = upload_input(inputs["text"])
        self.noise = upload_input(inputs["noise"])
        self.actions = torch.empty((d.chunk, d.action_dim), dtype=torch.float32, device=DEV)
        self.vel = torch.empty((cfg.steps, d.chunk, d.action_dim), dtype=torch.float32, device=DEV)
        self.hidden = torch.empty((cfg.seq, cfg.block.hidden), dtype=torch.int16, device=DEV) if with_hidden else None
        self.shape = lib.StepShape(n_images=cfg.n_images, n_text=cfg.n_text, chunk=d.chunk, action_dim=d.action_dim,
                                   steps=cfg.steps)
        self.io = lib.StepIO(images=None if self.images is None else self.images.data_ptr(), text=self.text.data_ptr(),
                             noise=self.noise.data_ptr(), actions=self.actions.data_ptr(),
                             hidden_out=None if self.hidden is None else self.hidden.data_ptr(),
                             velocities=self.vel.data_ptr())
        if n_stale is None:
            need = lib.vla_step_workspace_bytes(model, self.shape)
            assert need > 0, lib.vla_last_error()
            self.ws = workspace(need)
            st, self.plan = lib.vla_step_plan_create(model, self.shape, self.io, self.ws, need)
        else:   # a V-AEFusion plan: every pass is one control cycle
            need = lib.vla_step_fused_workspace_bytes(model, self.shape)
            assert need > 0, lib.vla_last_error()
            self.ws = workspace(need)
            st, self.plan = lib.vla_step_plan_create_fused(model, self.shape, self.io, n_stale, self.ws, need)
        lib.check(st)

    def load(self, inputs):
        """Refresh the static input buffers in place (the plan keeps their addresses)."""
        if self.images is not None:
            self.images.copy_(upload_input(inputs["image"]))
        self.text.copy_(upload_input(inputs["text"]))
        self.noise.copy_(upload_input(inputs["noise"]))

    def run(self, stream=0):
        lib.check(lib.vla_step_run(self.plan, stream))

    def capture(self, stream=0):
        lib.check(lib.vla_step_capture(self.plan, stream))

    def replay(self, stream=0):
        lib.check(lib.vla_step_replay(self.plan, stream))

    def outputs(self):
        torch.cuda.synchronize()
        out = {"actions": self.actions.cpu().numpy().astype(np.float64),
               "velocities": self.vel.cpu().numpy().astype(np.float64)}
        if self.hidden is not None:
            out["hidden"] = bf16_bits_to_float(self.hidden).astype(np.float64)
        return out

    def close(self):
        if self.plan:
            lib.vla_step_plan_destroy(self.plan)
            self.plan = None


def timed(label, fn):
    t = time.time()
    r = fn()
    say(f"  {label}: {time.time() - t:.1f}s")
    return r


class ProgressWeights(Weights):
    """Oracle weight access that prints which layer the oracle has reached
    (at most every few seconds), so a long full-size evaluation reports its
    own progress. Weights whose names start with ``keep_prefix`` (the action
    expert's, read once per Euler step) keep their float64 form after the
    first read."""

    def __init__(self, tensors, label: str, every_s: float = 5.0, keep_prefix: str = "dit."):
        super().__init__(tensors)
        self.keep_prefix = keep_prefix
        self.label = label
        self.every = every_s
        self.last = time.time()
        self.t0 = self.last
        self.n = 0

    def __getitem__(self, name: str):
        self.n += 1
        now = time.time()
        if now - self.last >= self.every:
            self.last = now
            say(f"  {self.label}: at {name} after {now - self.t0:.0f}s ({self.n} weight reads)")
        v = super().__getitem__(name)
        if name.startswith(self.keep_prefix):
            self._c[name] = v
        return v
